#!/usr/bin/env python3
"""Benchmark: Q4_K x int8 prefill GEMM on one MI355X.

Workload (one "step"): the small-model projection set at one 512-row ubatch --
hidden K=1024 -> fused QKV/gate N=4096 and MLP up/gate N=2x3584 (both read the
same hidden rows, so they share one activation quantisation), then down
K=3584 -> N=1024; all Q4_K weights (N(0, 0.02^2) packed), bf16 N(0,1)
activations, synthetic and seeded.  Each step runs the activation quantiser
twice and the tiled int8-MFMA GEMM three times, with inputs resident in HBM.

Printed: one JSON line with value = effective int8 TOPS of the step
(2*M*N*K summed over the three projections / step time), prefill tok/s,
the roofline of the dominant kernel (the tiled GEMM, timed per launch with HIP
events on its stream), the M=1 LM-head bandwidth (K=4096 -> N=152064, Q6_K)
and the CPU oracle timed on the host.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--lm-steps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the kernel is shown at one GPU's share of the work).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__.ensure_built()
    import synth
    import quantized_prefill_gemm_q8_amd as qg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

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

    gemm_events = []

    def gemm(g, ws, record):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        qg.qgemm_gemm_quantized(Wd[g.name], g.fmt, ws, M, g.N, g.K, y[g.name], stream,
                                qg.QG_PATH_TILED)
        if record:
            e1.record(stream)
            gemm_events.append((g.ops, e0, e1))

    def step(record=False):
        qg.qgemm_quantize_workspace(x_hidden, M, qkv.K, ws_h, stream)
        gemm(qkv, ws_h, record)
        gemm(up, ws_h, record)
        qg.qgemm_quantize_workspace(x_down, M, down.K, ws_d, stream)
        gemm(down, ws_d, record)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: whole steps, no per-kernel events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # timed region 2: the same steps with HIP events around every GEMM launch
    gemm_events.clear()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    g_ops = sum(o for o, _, _ in gemm_events)
    g_ms = sum(a.elapsed_time(b) for _, a, b in gemm_events)
    g_launches = len(gemm_events)
    gemm_tops = g_ops / (g_ms * 1e-3) / 1e12

    value = step_ops / (ms_per_step * 1e-3) / 1e12
    tok_s = M / (ms_per_step * 1e-3)

    # ---------------- LM head on the last token: M = 1, K = 4096 -> N = 152064, Q6_K
    lm = synth.CONFIGS[5][0]
    W_lm = to_dev(synth.make_weights(lm))
    x_lm = to_dev(synth.make_acts(lm))[0]
    ws_lm = qg.alloc_workspace(1, lm.K, dev)
    y_lm = torch.empty(lm.N, dtype=torch.float32, device=dev)
    for _ in range(5):
        qg.qgemm_lm_head(W_lm, lm.fmt, x_lm, lm.N, lm.K, y_lm, ws_lm, stream)
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.lm_steps):
        qg.qgemm_quantize_workspace(x_lm, 1, lm.K, ws_lm, stream)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qg.qgemm_gemm_quantized(W_lm, lm.fmt, ws_lm, 1, lm.N, lm.K, y_lm, stream, qg.QG_PATH_SKINNY)
        b.record(stream)
        ev.append((a, b))
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(args.lm_steps):
        qg.qgemm_lm_head(W_lm, lm.fmt, x_lm, lm.N, lm.K, y_lm, ws_lm, stream)
    c1.record(stream)
    torch.cuda.synchronize()
    lm_kernel_us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    lm_call_us = 1e3 * c0.elapsed_time(c1) / args.lm_steps
    lm_gbs = lm.w_bytes / (lm_kernel_us * 1e-6) / 1e9

    # ---------------- CPU oracle on the host (same step, whole workload, repeated)
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
        cpu = {"value": round(step_ops * reps / t_cpu / 1e12, 6), "unit": "TOPS (int8 ops)",
               "cores": cores, "kind": "oracle",
               "sample": f"the whole step (qkv_gate, up_gate, down at M=512, activation "
                         f"quantisation included) repeated {reps}x in {t_cpu:.1f} s",
               "tok_s": round(M * reps / t_cpu, 2)}

    out = {
        "metric": "effective int8 TOPS & prefill tok/s, Q4_K GEMM M=512 (+ GB/s at M=1 LM head)",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int8 -> int32, fp32 epilogue",
        "data": "synthetic (seeded N(0,0.02^2) weights packed to Q4_K, bf16 N(0,1) activations)",
        "config": {"workload": "small-model projection set, M=512: 1024->4096 + 1024->7168 "
                               "(shared hidden) + 3584->1024, Q4_K", "M": M,
                   "projections": [[g.K, g.N] for g in (qkv, up, down)]},
        "prefill_tok_s": round(tok_s, 1),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_q4k_kernel (tiled)",
                     "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 5),
                     "traffic": None, "launches": g_launches,
                     "avg_launch_us": round(1e3 * g_ms / g_launches, 3)},
        "lm_head": {"workload": "M=1, K=4096 -> N=152064, Q6_K (skinny path)",
                    "weight_bytes": lm.w_bytes, "kernel_us": round(lm_kernel_us, 3),
                    "call_us": round(lm_call_us, 3), "gbps": round(lm_gbs, 1),
                    "frac_hbm": round(lm_gbs / PEAK_HBM_GBS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
