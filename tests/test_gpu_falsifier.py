"""Timing falsifier for the benchmark's per-kernel rows (aprender issue #3598,
"EPIC E2 0.73: Verbs Are Fast", prior body, row 1): a delay planted in one
kernel must move that kernel's timing row and the step total, and leave the
other kernel's row where it was.  The rows are timed as the benchmark times
them: back-to-back calls between two HIP events on the calls' stream, the
least of several rounds.  The planted delay (qgemm_test_plant_delay) makes one
wave of the activation quantiser's first workgroup sleep a bounded number of
times; the output must not change.

Also the path log: QGEMM_TRACE=1 names every call's path and kernel on stderr
(aprender issue #5475, "Ask", item 2), checked in a child process that starts
with the variable set; and the read probe the decode GEMVs are quoted against
(qgemm_read_probe), whose time must grow with the bytes it reads."""
import os
import subprocess
import sys

import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(calls, stream, n=20, rounds=5):
    """Least microseconds per call of each callable over `rounds` rounds of n calls."""
    best = {k: float("inf") for k in calls}
    for _ in range(rounds):
        for k, fn in calls.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            best[k] = min(best[k], 1e3 * a.elapsed_time(b) / n)
    return best


def test_planted_delay_moves_only_its_row():
    M, K, N = 512, 4096, 4096
    W = to_dev(synth.pack(qg.QG_Q4_K, synth.normal(9201, (N, K), 0.0, 0.02)))
    x = to_dev(synth.to_bf16_bits(synth.student_t4(9202, (M, K))))
    ws = qg.alloc_workspace(M, K, DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream()

    def quant():
        qg.qgemm_quantize_workspace(x, M, K, ws, stream)

    def gemm():
        qg.qgemm_gemm_quantized(W, qg.QG_Q4_K, ws, M, N, K, y, stream)

    def step():
        quant()
        gemm()

    calls = {"quant": quant, "gemm": gemm, "step": step}
    for _ in range(200):  # let the clock settle
        step()
    torch.cuda.synchronize()
    y_base = y.clone()
    base = _rows(calls, stream)
    # about 40 us at 2 GHz (64 shader clocks per sleep)
    qg.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, 1250)
    try:
        step()
        torch.cuda.synchronize()
        assert torch.equal(y, y_base), "the planted delay changed the output"
        planted = _rows(calls, stream)
    finally:
        qg.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, 0)
    after = _rows(calls, stream)
    print(f"base {base}\nplanted {planted}\nafter {after}", flush=True)
    d = planted["quant"] - base["quant"]
    assert 15.0 < d < 400.0, f"the planted delay moved the quantiser row by {d:.2f} us"
    assert abs(planted["gemm"] - base["gemm"]) <= max(0.1 * base["gemm"], 3.0), "the GEMM row moved"
    assert abs((planted["step"] - base["step"]) - d) <= 0.25 * d + 3.0, "the step total did not move by d"
    assert abs(after["quant"] - base["quant"]) <= max(0.2 * base["quant"], 2.0), "the delay stayed"


def test_trace_names_path_and_kernel():
    cases = [(qg.QG_Q4_K, 64, 512, 256), (qg.QG_Q6_K, 1, 1024, 300), (qg.QG_Q4_K, 512, 4096, 4096)]
    script = (
        "import sys, torch, synth, quantized_prefill_gemm_q8_amd as qg\n"
        f"for fmt, M, K, N in {cases!r}:\n"
        "    W = torch.from_numpy(synth.pack(fmt, synth.normal(9301, (N, K), 0.0, 0.02))).cuda()\n"
        "    x = torch.from_numpy(synth.normal(9302, (M, K))).cuda()\n"
        "    qg.prefill(W, fmt, x, N)\n"
        "torch.cuda.synchronize()\n"
        "print('done', flush=True)\n")
    env = dict(os.environ, QGEMM_TRACE="1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("qgemm: ")]
    assert len(lines) == len(cases), r.stderr[-2000:]
    for (fmt, M, K, N), ln in zip(cases, lines):
        name = {qg.QG_Q4_K: "Q4_K", qg.QG_Q6_K: "Q6_K"}[fmt]
        skinny = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_AUTO).startswith("skinny_kernel<")
        want = (f"qgemm: gemm fmt={name} M={M} N={N} K={K} path={'skinny' if skinny else 'tiled'} "
                f"kernel={qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_AUTO)}")
        assert ln == want, (ln, want)


def test_read_probe_time_grows_with_bytes():
    """The read floor reads what it is given: four times the bytes take well over
    twice the time (a probe whose loads were dropped would not scale)."""
    stream = torch.cuda.Stream()
    small = torch.ones(64 << 20, dtype=torch.uint8, device=DEV)
    large = torch.ones(256 << 20, dtype=torch.uint8, device=DEV)
    qg.qgemm_read_probe(large, 0, stream)  # zero bytes: no launch, no error
    t = _rows({"small": lambda: qg.qgemm_read_probe(small, small.numel(), stream),
               "large": lambda: qg.qgemm_read_probe(large, large.numel(), stream)}, stream, n=10)
    print(f"read probe: 64 MiB {t['small']:.1f} us, 256 MiB {t['large']:.1f} us")
    assert t["large"] > 2.0 * t["small"], t

