"""Wait states before the inline-assembly LDS DMA loads (CPU only: compiles
device code to gfx950 assembly, runs nothing).

`global_load_lds_dwordx4` is issued from inline assembly (csrc/lds_stage.h),
which the compiler's hazard recognizer does not look into.  Its base address
reaches SGPRs through v_readfirstlane and its LDS address reaches M0 through an
SALU write; the hardware needs 5 wait states between a VALU write of an SGPR
and a vector-memory instruction reading it, and 1 between an SALU write of M0
and an LDS DMA.  Without them the load can use a stale base (a faulting kernel
variant did).  This test compiles the tiled kernels to assembly and checks
every DMA load against the instructions before it.  (The skinny kernel's DMA
path uses the same statement; its file takes two minutes to compile and is
left to the build.)"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_prefill_gemm_q8_amd", "csrc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S"]


def _wait_states(line):
    m = re.match(r"\s*s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def _sregs(spec):
    m = re.match(r"s\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def scan(text):
    """(number of DMA loads seen, list of hazards) in one assembly file."""
    lines = [ln for ln in text.splitlines()
             if ln.strip() and not ln.strip().startswith((";", "."))]
    seen, bad, func = 0, [], "?"
    for i, ln in enumerate(lines):
        if re.match(r"^_Z\S+:", ln):
            func = ln.split(":")[0]
        m = re.search(r"global_load_lds_dwordx4\s+v\d+,\s*(s\[\d+:\d+\]|off)", ln)
        if not m:
            continue
        seen += 1
        base = _sregs(m.group(1)) if m.group(1) != "off" else set()
        ws = 0
        for j in range(i - 1, max(-1, i - 12), -1):
            p = lines[j]
            if re.match(r"^\S", p):  # a label: the block starts here
                break
            mv = re.match(r"\s*(v_\w+)\s+(s\[\d+:\d+\]|s\d+)\b", p)
            if mv and ws < 5 and (_sregs(mv.group(2)) & base):
                bad.append(f"{func[:60]}: {mv.group(1)} writes {mv.group(2)} {ws} wait states before the DMA")
                break
            if re.match(r"\s*s_\w+\s+m0\b", p) and ws < 1:
                bad.append(f"{func[:60]}: M0 written {ws} wait states before the DMA")
            ws += _wait_states(p)
    return seen, bad


def test_scanner_finds_a_planted_hazard():
    asm = ("_Zk:\n\tv_readfirstlane_b32 s5, v17\n\tv_readfirstlane_b32 s4, v16\n"
           "\tglobal_load_lds_dwordx4 v46, s[4:5]\n")
    assert scan(asm)[1], "a base written right before the load must be reported"
    ok = ("_Zk:\n\tv_readfirstlane_b32 s5, v17\n\tv_readfirstlane_b32 s4, v16\n\ts_mov_b32 m0, s6\n"
          "\ts_nop 4\n\tglobal_load_lds_dwordx4 v46, s[4:5]\n")
    assert scan(ok) == (1, [])


def test_tiled_kernels_wait_before_every_dma(tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not found")
    procs = []
    for src in ("gemm_q4k.hip", "gemm_q6k.hip", "gemm_deq_f16.hip"):
        out = str(tmp_path / (src + ".s"))
        procs.append((src, out, subprocess.Popen(["hipcc", *FLAGS, os.path.join(CSRC, src), "-o", out],
                                                 stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    total = 0
    for src, out, p in procs:
        log = p.communicate(timeout=600)[0]
        assert p.returncode == 0, log[-2000:]
        seen, bad = scan(open(out).read())
        assert not bad, f"{src}: " + "; ".join(bad[:5])
        total += seen
    assert total > 100, f"only {total} DMA loads found: the scan did not see the kernels"
