#!/usr/bin/env python3
"""Benchmark: Q4_K x int8 prefill GEMM on one MI355X.

Workload (one "step"): the small-model projection set at one 512-row ubatch --
hidden K=1024 -> fused QKV/gate N=4096 and MLP up/gate N=2x3584 (both read the
same hidden rows, so they share one activation quantisation), then down
K=3584 -> N=1024; all Q4_K weights (N(0, 0.02^2) packed), bf16 N(0,1)
activations, synthetic and seeded.  Each step runs the activation quantiser
twice and the tiled int8-MFMA GEMM three times, with inputs resident in HBM.

Timing: library calls are issued back to back on one stream between two HIP
events on that stream.  The step and the long GEMMs are issued eagerly, one
call at a time (the host stays ahead of the GPU there; the step replayed from a
captured HIP graph is reported next to it); the decode-sized GEMVs and the LM
head, whose kernels are short enough for the host's per-call cost to pace an
eager loop, are captured once as a HIP graph and replayed.

Printed: one JSON line with value = effective int8 TOPS of the step
(2*M*N*K summed over the three projections / step time), prefill tok/s, the
roofline of the dominant kernel (the GEMM kernel with the largest share of the
step; its launches run back to back), the large-M headline
projections (K=4096 -> N=24576 Q4_K and K=12288 -> N=4096 Q6_K at M=512), the
decode-sized GEMV (M = 1 and 8) over every projection shape of the workloads,
the M=1 LM-head bandwidth (K=4096 -> N=152064, Q6_K), the other design branch
(weights dequantised to fp16 in the GEMM, fp16 matrix cores) and the per-256
activation-scale variant (Q4_K) beside the int8 method on every projection
shape, the fusions either side of the GEMM (RMSNorm -> quantiser, the gate+up
GEMM with the SwiGLU epilogue, and whole FFN blocks) against the unfused
chains, and the CPU oracle timed on the host.

--calib-copy-mib N additionally runs a plain elementwise copy kernel over
N MiB (read N, write N) three times: the reference dispatch for scaling HBM
byte counters taken with a profiler.

--pmc-summary FETCH_DB WRITE_DB OUT_JSON turns the databases of two
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of this script (with
--calib-copy-mib) into per-kernel HBM bytes per dispatch, scaled by what the
counters read for the copy kernel, stamped with a hash of the kernel sources;
a later benchmark run reports them as `roofline.traffic` only while the
sources still hash the same.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, vendor figure
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, vendor figure
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, vendor figure
COLD_BYTES = 600 * 1000 ** 2  # weight footprint that defeats the 256 MB MALL (cold-cache GEMV)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic_bench_workload.json")
CALIB_KERNEL = "neg_kernel"  # the copy kernel --calib-copy-mib launches


def source_hash() -> str:
    """sha256 over the library's kernel and header sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_prefill_gemm_q8_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    files.append(os.path.join(ROOT, "include", "qgemm.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_kernel_name(name: str) -> str:
    """'void qg::gemm_x<1, 2>(args)' -> 'gemm_x<1, 2>' (the form qgemm_kernel_name returns)."""
    name = name.split("(")[0].strip()
    if name.startswith("void "):
        name = name[5:]
    if name.startswith("qg::"):
        name = name[4:]
    return name


def pmc_summary(fetch_db: str, write_db: str, out_json: str, calib_mib: int) -> None:
    import sqlite3
    per = {}
    for db, counter in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        con = sqlite3.connect(db)
        rows = con.execute("select name, dispatch_id, counter_value from pmc_events "
                           "where counter_name = ?", (counter,)).fetchall()
        disp = {}
        for name, did, v in rows:
            key = (name, did)
            disp[key] = disp.get(key, 0.0) + float(v)
        for (name, _), v in disp.items():
            d = per.setdefault(name, {}).setdefault(counter, [])
            d.append(v)
    calib = [n for n in per if CALIB_KERNEL in n]
    if not calib:
        raise SystemExit("no calibration copy kernel in the databases (run with --calib-copy-mib)")
    cbytes = calib_mib * (1 << 20)
    cf = per[calib[0]]
    f_scale = cbytes / (sum(cf["FETCH_SIZE"]) / len(cf["FETCH_SIZE"]) * 1024.0)
    w_scale = cbytes / (sum(cf["WRITE_SIZE"]) / len(cf["WRITE_SIZE"]) * 1024.0)
    out = {"source_sha256": source_hash(), "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "calib_bytes": cbytes, "kernels": {}}
    for name, d in per.items():
        if "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        fk = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
        wk = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
        out["kernels"][short_kernel_name(name)] = {
            "dispatches": len(d["FETCH_SIZE"]), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
            "read_bytes": round(fk * 1024 * f_scale), "write_bytes": round(wk * 1024 * w_scale)}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")


def traffic_for(kernel: str):
    """HBM bytes per dispatch of `kernel` from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k["read_bytes"] + k["write_bytes"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--lm-steps", type=int, default=50)    # 0: skip the LM head
    p.add_argument("--big-steps", type=int, default=30)   # 0: skip the large-M GEMMs
    p.add_argument("--gemv-steps", type=int, default=200)  # 0: skip the decode GEMV table
    p.add_argument("--set-steps", type=int, default=10)   # 0: skip the config 3/4 projection sets
    p.add_argument("--branch-steps", type=int, default=5)  # 0: skip the design-variants table
    p.add_argument("--fusion-steps", type=int, default=5)  # 0: skip the fusions table
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calib-copy-mib", type=int, default=0)
    p.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "OUT_JSON"))
    p.add_argument("--single", metavar="WORKLOAD",
                   help="time one workload GEMM only (e.g. c4_gate_up_M512) and print its line")
    p.add_argument("--single-branch", choices=("int8", "f16"), default="int8",
                   help="with --single: the int8 method (default) or the fp16 design branch")
    return p.parse_args()


def run_single(name: str, steps: int, branch: str = "int8") -> None:
    """Quantise once, then time `steps` back-to-back launches of one workload GEMM
    (branch "f16": whole calls of the fp16 design branch, conversion included)."""
    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__.ensure_built()
    import synth
    import quantized_prefill_gemm_q8_amd as qg
    allg = {f"c{c}_{g.name}": g for c in synth.CONFIGS for g in synth.CONFIGS[c]}
    if name not in allg:
        raise SystemExit(f"unknown workload {name}; one of: {', '.join(sorted(allg))}")
    g = allg[name]
    dev = torch.device("cuda:0")
    W = torch.from_numpy(synth.make_weights(g)).to(dev)
    xb = synth.make_acts(g)
    x = torch.from_numpy(xb.view(np.int16) if xb.dtype == np.uint16 else xb).to(dev)
    if xb.dtype == np.uint16:
        x = x.view(torch.bfloat16)
    y = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
    if branch == "f16":
        ws = torch.empty(qg.qgemm_deq_f16_workspace_bytes(g.M, g.K), dtype=torch.uint8, device=dev)
        call = lambda: qg.qgemm_prefill_deq_f16(W, g.fmt, x, g.M, g.N, g.K, y, ws)
        kname = qg.qgemm_deq_f16_kernel_name(g.fmt, g.M, g.N, g.K)
    else:
        ws = qg.alloc_workspace(g.M, g.K, dev)
        qg.qgemm_quantize_workspace(x, g.M, g.K, ws)
        call = lambda: qg.qgemm_gemm_quantized(W, g.fmt, ws, g.M, g.N, g.K, y)
        kname = qg.qgemm_kernel_name(g.fmt, g.M, g.N, g.K)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    print(json.dumps({"workload": name, "branch": branch, "shape": [g.M, g.K, g.N],
                      "fmt": "Q4_K" if g.fmt == 0 else "Q6_K",
                      "kernel": kname, "avg_launch_us": round(us, 3),
                      "tops": round(g.ops / (us * 1e-6) / 1e12, 2),
                      "gbps_weights": round(g.w_bytes / (us * 1e-6) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, calib_mib=args.calib_copy_mib or 1024)
        return
    if args.single:
        run_single(args.single, max(1, min(args.steps, 50)), args.single_branch)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the kernel is shown at one GPU's share of the work).", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__.ensure_built()
    import synth
    import quantized_prefill_gemm_q8_amd as qg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # every timed launch goes to one non-default stream: HIP graphs are captured
    # on it and replayed on it, and the timing events are recorded on it
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def capture(fn, n):
        """A HIP graph of n back-to-back calls fn() on `stream` (the library's
        launches are recorded, not run; nothing is allocated inside)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                fn()
        return g

    def time_replays(g, replays):
        """ms for `replays` back-to-back replays of g, between two events on `stream`."""
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(replays):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def per_graph(total):
        """calls per captured graph and replays for `total` timed calls"""
        n = min(total, 50)
        return n, max(1, (total + n - 1) // n)

    # ---------------- workload: the small-model projection set, M = 512
    qkv, up, down = synth.CONFIGS[2]
    M = qkv.M
    Wd = {g.name: to_dev(synth.make_weights(g)) for g in (qkv, up, down)}
    x_hidden = to_dev(synth.make_acts(qkv))     # shared by qkv_gate and up_gate
    x_down = to_dev(synth.make_acts(down))
    ws_h = qg.alloc_workspace(M, qkv.K, dev)
    ws_d = qg.alloc_workspace(M, down.K, dev)
    y = {g.name: torch.empty((M, g.N), dtype=torch.float32, device=dev) for g in (qkv, up, down)}
    step_ops = sum(g.ops for g in (qkv, up, down))
    kname = {g.name: qg.qgemm_kernel_name(g.fmt, M, g.N, g.K, qg.QG_PATH_TILED)
             for g in (qkv, up, down)}

    # ---------------- CPU oracle on the host (same step, whole workload, repeated),
    # timed before any GPU work of this process
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        host = {g.name: (synth.make_weights(g), synth.make_acts(g)) for g in (qkv, up, down)}
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 1000:
            s0 = time.perf_counter()
            for g in (qkv, up, down):
                Wn, xn = host[g.name]
                oracle.gemm(g.fmt, Wn, xn, g.N)
            t_cpu += time.perf_counter() - s0
            reps += 1
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        cpu = {"value": round(step_ops * reps / t_cpu / 1e12, 6), "unit": "TOPS",
               "cores": cores, "kind": "oracle",
               "sample": f"the whole step (qkv_gate, up_gate, down at M=512; activation "
                         f"quantisation included) repeated {reps}x in {t_cpu:.1f} s",
               "tok_s": round(M * reps / t_cpu, 2)}


    def gemm(g, ws):
        qg.qgemm_gemm_quantized(Wd[g.name], g.fmt, ws, M, g.N, g.K, y[g.name], stream,
                                qg.QG_PATH_TILED)

    def step():
        qg.qgemm_quantize_workspace(x_hidden, M, qkv.K, ws_h, stream)
        gemm(qkv, ws_h)
        gemm(up, ws_h)
        qg.qgemm_quantize_workspace(x_down, M, down.K, ws_d, stream)
        gemm(down, ws_d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: whole steps, issued eagerly, no per-kernel events
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # per-step distribution: the same steps with an event pair around each
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in evs)

    def pct(xs, q):
        return xs[min(len(xs) - 1, int(q * len(xs)))]
    # the same steps replayed from a captured HIP graph (for reference)
    per, replays = per_graph(args.steps)
    g_step = capture(step, per)
    time_replays(g_step, 1)
    graph_ms_per_step = time_replays(g_step, replays) / (per * replays)
    del g_step

    # timed region 2: per GEMM kernel, its launches of one step run back to back
    # (same arguments, same stream) between two HIP events, repeated `steps`
    # times: the average launch duration with no per-launch event in between
    groups = {}
    for g, ws in ((qkv, ws_h), (up, ws_h), (down, ws_d)):
        groups.setdefault(kname[g.name], []).append((g, ws))
    per_kernel = {}
    for name, members in groups.items():
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(args.steps):
            for g, ws in members:
                gemm(g, ws)
        b.record(stream)
        torch.cuda.synchronize()
        per_kernel[name] = {"ops": args.steps * sum(g.ops for g, _ in members),
                            "ms": a.elapsed_time(b), "launches": args.steps * len(members)}
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
    dk = per_kernel[dom]
    dom_tops = dk["ops"] / (dk["ms"] * 1e-3) / 1e12
    gemm_ms = sum(d["ms"] for d in per_kernel.values()) / args.steps

    value = step_ops / (ms_per_step * 1e-3) / 1e12
    tok_s = M / (ms_per_step * 1e-3)

    # ---------------- large-M headline projections (one GEMM each, M = 512)
    big = {}
    for g in (synth.CONFIGS[4][0], synth.CONFIGS[4][1]) if args.big_steps > 0 else ():
        Wb = to_dev(synth.make_weights(g))
        xb = to_dev(synth.make_acts(g))
        wsb = qg.alloc_workspace(g.M, g.K, dev)
        yb = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
        qg.qgemm_quantize_workspace(xb, g.M, g.K, wsb, stream)

        for _ in range(5):
            qg.qgemm_gemm_quantized(Wb, g.fmt, wsb, g.M, g.N, g.K, yb, stream)
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(args.big_steps):
            qg.qgemm_gemm_quantized(Wb, g.fmt, wsb, g.M, g.N, g.K, yb, stream)
        b.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / args.big_steps
        tops = g.ops / (us * 1e-6) / 1e12
        big[f"{g.name}"] = {"shape": f"M={g.M} K={g.K} N={g.N} "
                                     f"{'Q4_K' if g.fmt == qg.QG_Q4_K else 'Q6_K'}",
                            "kernel": qg.qgemm_kernel_name(g.fmt, g.M, g.N, g.K),
                            "avg_launch_us": round(us, 2), "tops": round(tops, 1),
                            "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4)}
        del Wb, xb, wsb, yb

    # ---------------- one layer's projection set of the mid-size and long-prompt
    # configurations at each prompt length: quantise each input, run each GEMM
    # (the weights of a configuration do not depend on M); prefill tok/s per layer
    sets = {}
    for cfg in (3, 4) if args.set_steps > 0 else ():
        gs = synth.CONFIGS[cfg]
        Ws = {}
        for Mset in sorted({g.M for g in gs}):
            members = [g for g in gs if g.M == Mset]
            bufs = []
            for g in members:
                key = (g.K, g.N, g.fmt)
                if key not in Ws:
                    Ws[key] = to_dev(synth.make_weights(g))
                xs = to_dev(synth.make_acts(g))
                wss = qg.alloc_workspace(g.M, g.K, dev)
                ys = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
                bufs.append((g, Ws[key], xs, wss, ys))

            def set_step(bufs=bufs):
                for g, Wm, xs, wss, ys in bufs:
                    qg.qgemm_quantize_workspace(xs, g.M, g.K, wss, stream)
                    qg.qgemm_gemm_quantized(Wm, g.fmt, wss, g.M, g.N, g.K, ys, stream)
            for _ in range(2):
                set_step()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(args.set_steps):
                set_step()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.set_steps
            ops = sum(g.ops for g in members)
            sets[f"config{cfg}_M{Mset}"] = {
                "projections": [f"{g.K}->{g.N} {'Q4_K' if g.fmt == qg.QG_Q4_K else 'Q6_K'}" for g in members],
                "ms_per_layer": round(ms, 4), "prefill_tok_s": round(Mset / (ms * 1e-3), 1),
                "tops": round(ops / (ms * 1e-3) / 1e12, 2)}
            del bufs
        del Ws
    torch.cuda.empty_cache()

    # ---------------- the measured design variants beside the int8 method, per
    # projection shape, each timed as whole calls back to back (best of three
    # interleaved rounds): the int8 method
    # (quantiser + GEMM), per-256 activation scales (Q4_K: quantiser + GEMM) and
    # the other design branch (x -> binary16 + GEMM on fp16 matrix cores)
    variants = {}
    for cfg in (2, 3, 4) if args.branch_steps > 0 else ():
        for g in synth.CONFIGS[cfg]:
            Wb = to_dev(synth.make_weights(g))
            xb = to_dev(synth.make_acts(g))
            yb = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
            ws8 = qg.alloc_workspace(g.M, g.K, dev)
            ws16 = torch.empty(qg.qgemm_deq_f16_workspace_bytes(g.M, g.K), dtype=torch.uint8,
                               device=dev)
            calls = {
                "int8": lambda: qg.qgemm_prefill(Wb, g.fmt, xb, g.M, g.N, g.K, yb, ws8, stream),
                "f16": lambda: qg.qgemm_prefill_deq_f16(Wb, g.fmt, xb, g.M, g.N, g.K, yb, ws16,
                                                        stream)}
            if g.fmt == qg.QG_Q4_K:
                calls["a256"] = lambda: qg.qgemm_prefill_a256(Wb, g.fmt, xb, g.M, g.N, g.K, yb, ws8,
                                                              stream)
                # the same shape with Q5_K and Q8_0 weights (int8 method)
                W5 = to_dev(synth.make_weights(dataclasses.replace(g, fmt=qg.QG_Q5_K)))
                calls["q5k"] = lambda: qg.qgemm_prefill(W5, qg.QG_Q5_K, xb, g.M, g.N, g.K, yb, ws8, stream)
                W8 = to_dev(synth.make_weights(dataclasses.replace(g, fmt=qg.QG_Q8_0)))
                calls["q80"] = lambda: qg.qgemm_prefill(W8, qg.QG_Q8_0, xb, g.M, g.N, g.K, yb, ws8, stream)
            # interleaved rounds, the best of three per variant (clocks drift
            # under sustained load; interleaving keeps the comparison fair)
            us = {}
            for fn in calls.values():
                for _ in range(2):
                    fn()
            for _ in range(3):
                for k, fn in calls.items():
                    a, b = ev(), ev()
                    a.record(stream)
                    for _ in range(args.branch_steps):
                        fn()
                    b.record(stream)
                    torch.cuda.synchronize()
                    us[k] = min(us.get(k, 1e30), 1e3 * a.elapsed_time(b) / args.branch_steps)
            rate = lambda k: round(g.ops / (us[k] * 1e-6) / 1e12, 1)
            row = {"shape": f"M={g.M} K={g.K} N={g.N} {'Q4_K' if g.fmt == qg.QG_Q4_K else 'Q6_K'}",
                   "int8_us": round(us["int8"], 2), "int8_tops": rate("int8")}
            if "q5k" in us:
                row.update({"q5k_us": round(us["q5k"], 2), "q5k_tops": rate("q5k"),
                            "q5k_kernel": qg.qgemm_kernel_name(qg.QG_Q5_K, g.M, g.N, g.K),
                            "q80_us": round(us["q80"], 2), "q80_tops": rate("q80"),
                            "q80_kernel": qg.qgemm_kernel_name(qg.QG_Q8_0, g.M, g.N, g.K)})
                del W5, W8
            if "a256" in us:
                row.update({"a256_us": round(us["a256"], 2), "a256_tops": rate("a256"),
                            "a256_kernel": qg.qgemm_kernel_name_a256(g.fmt, g.M, g.N, g.K),
                            "a256_over_int8_speed": round(us["int8"] / us["a256"], 3)})
            row.update({"f16_us": round(us["f16"], 2), "f16_tflops": rate("f16"),
                        "f16_frac_fp16_peak": round(rate("f16") / PEAK_FP16_TFLOPS, 4),
                        "f16_kernel": qg.qgemm_deq_f16_kernel_name(g.fmt, g.M, g.N, g.K),
                        "f16_over_int8_speed": round(us["int8"] / us["f16"], 3)})
            variants[f"c{cfg}_{g.name}"] = row
            del Wb, xb, yb, ws8, ws16
    torch.cuda.empty_cache()

    # ---------------- fusions either side of the GEMM, per gate+up projection of the
    # workloads (its 2F weight rows read as the stacked gate and up tensors) and
    # per FFN block (gate+up, SwiGLU, down): unfused = quantiser, GEMM to fp32
    # [M][2F], SwiGLU kernel (and the down projection's quantiser + GEMM); fused
    # = RMSNorm -> quantiser, gate+up GEMM with the SwiGLU epilogue writing bf16
    # (and the same down projection).  The fused chain also does the norm, which
    # the unfused one leaves out, so its advantage is understated.  Each call
    # sequence is timed back to back, best of three interleaved rounds.
    fusions = {}
    for cfg in (2, 3, 4) if args.fusion_steps > 0 else ():
        ups = [g for g in synth.CONFIGS[cfg] if (g.name == "up_gate" or g.name.startswith("gate_up"))
               and g.fmt == qg.QG_Q4_K]
        for g in ups:
            down = next(d for d in synth.CONFIGS[cfg] if d.name.startswith("down") and d.M == g.M)
            if down.K == g.N:
                # one of the two K->F tensors (the down projection reads F = N): stack it
                # with a second one of the same recipe as the up tensor
                F = g.N
                Wnp = np.concatenate([synth.make_weights(g),
                                      synth.pack(g.fmt, synth.normal(g.w_seed + 5, (g.N, g.K), 0.0, 0.02))])
            else:
                F = g.N // 2                       # already the stacked [gate; up] tensor
                assert down.K == F
                Wnp = synth.make_weights(g)
            gu_ops = 2 * g.M * 2 * F * g.K
            Wb = to_dev(Wnp)
            del Wnp
            xb = to_dev(synth.make_acts(g))
            gn = to_dev(synth.normal(7000 + g.K, (g.K,), 1.0, 0.25))
            ws = torch.empty(qg.qgemm_swiglu_workspace_bytes(g.fmt, g.M, F, g.K), dtype=torch.uint8,
                             device=dev)
            y2 = torch.empty((g.M, 2 * F), dtype=torch.float32, device=dev)
            hb = torch.empty((g.M, F), dtype=torch.bfloat16, device=dev)
            Wd = to_dev(synth.make_weights(down))
            wsd = qg.alloc_workspace(down.M, down.K, dev)
            yd = torch.empty((down.M, down.N), dtype=torch.float32, device=dev)
            calls = {
                "quant": lambda: qg.qgemm_quantize_workspace(xb, g.M, g.K, ws, stream),
                "rmsnorm_quant": lambda: qg.qgemm_rmsnorm_quantize_workspace(xb, gn, 1e-6, g.M, g.K, ws,
                                                                             stream),
                "gemm_fp32": lambda: qg.qgemm_gemm_quantized(Wb, g.fmt, ws, g.M, 2 * F, g.K, y2, stream),
                "gemm_swiglu": lambda: qg.qgemm_gemm_quantized_swiglu(Wb, g.fmt, ws, g.M, F, g.K, hb, stream),
                "swiglu": lambda: qg.qgemm_swiglu(y2, g.M, F, hb, stream)}

            def unfused():
                calls["quant"]()
                calls["gemm_fp32"]()
                calls["swiglu"]()

            def fused():
                calls["rmsnorm_quant"]()
                calls["gemm_swiglu"]()
            calls["unfused_chain"], calls["fused_chain"] = unfused, fused

            def down_proj():
                qg.qgemm_prefill(Wd, down.fmt, hb, down.M, down.N, down.K, yd, wsd, stream)
            calls["ffn_unfused"] = lambda: (unfused(), down_proj())
            calls["ffn_fused"] = lambda: (fused(), down_proj())
            us = {}
            for fn in calls.values():
                for _ in range(2):
                    fn()
            for _ in range(3):
                for k, fn in calls.items():
                    a, b = ev(), ev()
                    a.record(stream)
                    for _ in range(args.fusion_steps):
                        fn()
                    b.record(stream)
                    torch.cuda.synchronize()
                    us[k] = min(us.get(k, 1e30), 1e3 * a.elapsed_time(b) / args.fusion_steps)
            rms_bytes = g.M * g.K * 2 + g.K * 4 + g.M * g.K + g.M * (g.K // 32) * (4 + 4 + 4 + 6)
            ops = gu_ops + down.ops
            row = {"shape": f"M={g.M} K={g.K} gate+up 2x{F} Q4_K, down {down.K}->{down.N} "
                            f"{'Q4_K' if down.fmt == qg.QG_Q4_K else 'Q6_K'}",
                   "fused_kernel": qg.qgemm_kernel_name_swiglu(g.fmt, g.M, F, g.K),
                   **{f"{k}_us": round(v, 2) for k, v in us.items()},
                   "gemm_swiglu_tops": round(gu_ops / (us["gemm_swiglu"] * 1e-6) / 1e12, 1),
                   "gemm_swiglu_over_gemm_fp32_speed": round(us["gemm_fp32"] / us["gemm_swiglu"], 3),
                   "fused_over_unfused_chain_speed": round(us["unfused_chain"] / us["fused_chain"], 3),
                   "output_bytes_fp32_vs_bf16": [g.M * 2 * F * 4, g.M * F * 2],
                   "rmsnorm_quant_gbps": round(rms_bytes / (us["rmsnorm_quant"] * 1e-6) / 1e9, 1),
                   "ffn_fused_tok_s": round(g.M / (us["ffn_fused"] * 1e-6), 1),
                   "ffn_fused_tops": round(ops / (us["ffn_fused"] * 1e-6) / 1e12, 1),
                   "ffn_fused_over_unfused_speed": round(us["ffn_unfused"] / us["ffn_fused"], 3)}
            fusions[f"c{cfg}_{g.name}"] = row
            del Wb, xb, gn, ws, y2, hb, Wd, wsd, yd
    torch.cuda.empty_cache()

    # ---------------- decode-sized GEMV over every projection shape of the workloads
    # (M = 1 and M = 8 rows; weight bytes / kernel time against 8 TB/s)
    gemv = {}
    seen = set()
    fmt_name = {qg.QG_Q4_K: "Q4_K", qg.QG_Q5_K: "Q5_K", qg.QG_Q6_K: "Q6_K", qg.QG_Q8_0: "Q8_0"}
    # every Q4_K projection also as Q5_K (the format the pages' decode-GEMV ticket
    # finds slowest) and Q8_0: the same shape and weight recipe
    gemv_shapes = [g2 for cfg in ((2, 3, 4) if args.gemv_steps > 0 else ()) for g in synth.CONFIGS[cfg]
                   for g2 in ([g] + [dataclasses.replace(g, fmt=f) for f in (qg.QG_Q5_K, qg.QG_Q8_0)]
                              if g.fmt == qg.QG_Q4_K else [g])]
    for g in gemv_shapes:
        key = (g.K, g.N, g.fmt)
        if key in seen:
            continue
        seen.add(key)
        Wg = to_dev(synth.make_weights(g))
        xg = to_dev(synth.make_acts(g, rows=8))
        for Mg in (1, 8):
            wsg = qg.alloc_workspace(Mg, g.K, dev)
            yg = torch.empty((Mg, g.N), dtype=torch.float32, device=dev)
            qg.qgemm_quantize_workspace(xg[:Mg].contiguous(), Mg, g.K, wsg, stream)

            def gemv_call(g=g, Wg=Wg, wsg=wsg, yg=yg, Mg=Mg):
                qg.qgemm_gemm_quantized(Wg, g.fmt, wsg, Mg, g.N, g.K, yg, stream)
            for _ in range(3):
                gemv_call()
            n, r = per_graph(args.gemv_steps)
            gg = capture(gemv_call, n)
            time_replays(gg, 1)
            us = 1e3 * time_replays(gg, r) / (n * r)
            del gg
            # cold: launches rotate through copies of W whose footprint exceeds
            # twice the 256 MB MALL, so every launch streams its weights from HBM
            copies = [Wg] + [Wg.clone() for _ in range(max(1, -(-COLD_BYTES // g.w_bytes)) - 1)]
            ring = iter(range(1 << 30))

            def gemv_cold(g=g, wsg=wsg, yg=yg, Mg=Mg, copies=copies, ring=ring):
                qg.qgemm_gemm_quantized(copies[next(ring) % len(copies)], g.fmt, wsg, Mg, g.N, g.K,
                                        yg, stream)
            nc = max(n, len(copies))
            gc = capture(gemv_cold, nc)
            time_replays(gc, 1)
            us_cold = 1e3 * time_replays(gc, r) / (nc * r)
            del gc, copies
            gbs = g.w_bytes / (us * 1e-6) / 1e9
            gbs_cold = g.w_bytes / (us_cold * 1e-6) / 1e9
            gemv[f"K={g.K} N={g.N} {fmt_name[g.fmt]} M={Mg}"] = {
                "kernel": qg.qgemm_kernel_name(g.fmt, Mg, g.N, g.K),
                "weight_bytes": g.w_bytes, "avg_launch_us": round(us, 2),
                "gbps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                "cold_avg_launch_us": round(us_cold, 2), "cold_gbps": round(gbs_cold, 1),
                "cold_frac_hbm": round(gbs_cold / PEAK_HBM_GBS, 4)}
        del Wg, xg

    # ---------------- LM head on the last token: M = 1, K = 4096 -> N = 152064, Q6_K
    lm_out = None
    if args.lm_steps > 0:
        lm = synth.CONFIGS[5][0]
        W_lm = to_dev(synth.make_weights(lm))
        x_lm = to_dev(synth.make_acts(lm))[0]
        ws_lm = qg.alloc_workspace(1, lm.K, dev)
        y_lm = torch.empty(lm.N, dtype=torch.float32, device=dev)
        def lm_call():
            qg.qgemm_lm_head(W_lm, lm.fmt, x_lm, lm.N, lm.K, y_lm, ws_lm, stream)

        def lm_gemm():
            qg.qgemm_gemm_quantized(W_lm, lm.fmt, ws_lm, 1, lm.N, lm.K, y_lm, stream,
                                    qg.QG_PATH_SKINNY)
        # warm-up long enough (about 20 ms) for clocks to settle after the
        # lighter work before it
        for _ in range(200):
            lm_call()
        torch.cuda.synchronize()
        qg.qgemm_quantize_workspace(x_lm, 1, lm.K, ws_lm, stream)
        n, r = per_graph(args.lm_steps)
        ga, gc = capture(lm_gemm, n), capture(lm_call, n)
        time_replays(ga, 1)
        lm_kernel_us = 1e3 * time_replays(ga, r) / (n * r)
        time_replays(gc, 1)
        lm_call_us = 1e3 * time_replays(gc, r) / (n * r)
        del ga, gc
        lm_gbs = lm.w_bytes / (lm_kernel_us * 1e-6) / 1e9
        del W_lm
        lm_out = {"workload": "M=1, K=4096 -> N=152064, Q6_K (skinny path)",
                  "kernel": qg.qgemm_kernel_name(lm.fmt, 1, lm.N, lm.K),
                  "weight_bytes": lm.w_bytes, "kernel_us": round(lm_kernel_us, 3),
                  "call_us": round(lm_call_us, 3), "gbps": round(lm_gbs, 1),
                  "frac_hbm": round(lm_gbs / PEAK_HBM_GBS, 4),
                  "traffic": traffic_for(qg.qgemm_kernel_name(lm.fmt, 1, lm.N, lm.K))}

    # ---------------- optional: plain copy kernel of known size (profiler counter scale)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "effective int8 TOPS & prefill tok/s, Q4_K GEMM M=512 (+ GB/s at M=1 LM head)",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "graph_ms_per_step": round(graph_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,0.02^2) weights packed to Q4_K, bf16 N(0,1) activations)",
        "config": {"workload": "small-model projection set, M=512: 1024->4096 + 1024->7168 "
                               "(shared hidden) + 3584->1024, Q4_K", "M": M,
                   "projections": [[g.K, g.N] for g in (qkv, up, down)]},
        "prefill_tok_s": round(tok_s, 1),
        "gemm_ms_per_step": round(gemm_ms, 5),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "kernel": dom,
                     "achieved": round(dom_tops, 3), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tops / PEAK_INT8_TOPS, 5),
                     "traffic": traffic_for(dom), "launches": dk["launches"],
                     "avg_launch_us": round(1e3 * dk["ms"] / dk["launches"], 3),
                     "ops_per_launch": dk["ops"] // dk["launches"]},
        "gemm_kernels": {k: {"launches": d["launches"],
                             "avg_launch_us": round(1e3 * d["ms"] / d["launches"], 3),
                             "tops": round(d["ops"] / (d["ms"] * 1e-3) / 1e12, 2)}
                         for k, d in per_kernel.items()},
        "step_ms_p10_p50_p90": [round(pct(step_ms, 0.1), 5), round(pct(step_ms, 0.5), 5),
                                round(pct(step_ms, 0.9), 5)],
        "large_m": big,
        "projection_sets": sets,
        "decode_gemv": gemv,
        "lm_head": lm_out,
        "design_variants": variants,
        "fusions": fusions,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
