"""Build recipe for libqgemm.so: hipcc for gfx950, one object per source, in-tree.

Each build also writes libqgemm.so.json beside the library: a sha256 over the
kernel and header sources it was built from (and the git commit, when the tree
is a checkout).  The binding refuses a library whose sources have changed
since, so a forgotten rebuild cannot pass tests against stale kernels.
"""
from __future__ import annotations

import hashlib
import json
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqgemm.so")
INFO = LIB + ".json"
HEADER = os.path.join(os.path.dirname(PKG), "include", "qgemm.h")
SOURCES = ["act_quant.hip", "gemm_q4k.hip", "gemm_q6k.hip", "gemm_probe.hip", "gemm_skinny.hip",
           "gemm_deq_f16.hip", "swiglu.hip", "dequant.hip", "clock.hip", "noalloc.hip", "api.hip"]
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def source_sha256() -> str:
    """sha256 over every file of csrc/ and the public header."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC))
    files.append(HEADER)
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _git_sha() -> str | None:
    try:
        r = subprocess.run(["git", "-C", os.path.dirname(PKG), "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        return r.stdout.strip() or None if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def build_info() -> dict:
    """What the last build recorded ({} when there is none)."""
    try:
        with open(INFO) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return {}


def is_stale() -> bool:
    """True when the library was built from other sources than the tree holds."""
    return build_info().get("source_sha256") != source_sha256()


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((cmd, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    digest = source_sha256()
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    with open(INFO + ".tmp", "w") as fh:
        json.dump({"source_sha256": digest, "git_sha": _git_sha()}, fh)
    os.replace(INFO + ".tmp", INFO)
    return LIB
