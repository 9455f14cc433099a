"""Seeded synthetic inputs for the Q4_K / Q6_K x int8 prefill GEMM.

Holds no GEMM arithmetic.  It writes the weight blocks and activation rows
that both the CPU oracle and the GPU library consume, plus the workload
recipes (shapes, distributions, seeds) the tests and the benchmark share.

The C core (``synth.c``) is built in-tree with gcc into ``libsynth.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

Q4_K = 0
Q6_K = 1
Q5_K = 2
Q8_0 = 3
F32 = 0
BF16 = 1
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q5_K: 176, Q8_0: 272}   # bytes per 256 values


def build() -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP, no fast-math)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_u64.argtypes = [u64, u64]
        lib.synth_u64.restype = u64
        lib.synth_uniform_f64.argtypes = [u64, i64, vp]
        lib.synth_normal_f32.argtypes = [u64, i64, dbl, dbl, vp]
        lib.synth_outliers_f32.argtypes = [u64, i64, dbl, dbl, vp]
        lib.synth_student_t4_f32.argtypes = [u64, i64, vp]
        lib.synth_rmsnorm_rows_f32.argtypes = [vp, i64, i64, dbl]
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.synth_pack_q4k.argtypes = [vp, i64, i64, vp]
        lib.synth_pack_q5k.argtypes = [vp, i64, i64, vp]
        lib.synth_pack_q6k.argtypes = [vp, i64, i64, vp]
        lib.synth_pack_q80.argtypes = [vp, i64, i64, vp]
        lib.synth_random_blocks.argtypes = [u64, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, vp]
        for f in ("synth_uniform_f64", "synth_normal_f32", "synth_outliers_f32",
                  "synth_student_t4_f32", "synth_rmsnorm_rows_f32", "synth_f32_to_bf16",
                  "synth_pack_q4k", "synth_pack_q6k", "synth_random_blocks"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def u64(seed: int, i: int) -> int:
    return int(_load().synth_u64(seed, i))


def uniform(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform_f64(seed, n, _ptr(out))
    return out


def normal(seed: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, out.size, mean, std, _ptr(out))
    return out


def add_outliers(x: np.ndarray, mask_seed: int, prob: float, factor: float) -> np.ndarray:
    _load().synth_outliers_f32(mask_seed, x.size, prob, factor, _ptr(x))
    return x


def student_t4(seed: int, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_student_t4_f32(seed, out.size, _ptr(out))
    return out


def rmsnorm_rows(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    assert x.ndim == 2 and x.dtype == np.float32
    _load().synth_rmsnorm_rows_f32(_ptr(x), x.shape[0], x.shape[1], eps)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().synth_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def pack(fmt: int, w: np.ndarray) -> np.ndarray:
    """Pack float weights [N x K] into GGUF blocks; returns uint8 [N, K/256*bytes]."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    assert K % 256 == 0
    out = np.empty((N, K // 256 * BLOCK_BYTES[fmt]), np.uint8)
    fn = {Q4_K: _load().synth_pack_q4k, Q5_K: _load().synth_pack_q5k, Q6_K: _load().synth_pack_q6k,
          Q8_0: _load().synth_pack_q80}[fmt]
    fn(_ptr(w), N, K, _ptr(out))
    return out


def random_blocks(fmt: int, N: int, K: int, seed: int, emin: int = 1, emax: int = 14,
                  allow_negative: bool = True) -> np.ndarray:
    """Random legal blocks (random bits, finite binary16 scales)."""
    assert K % 256 == 0 and 0 <= emin <= emax <= 30
    out = np.empty((N, K // 256 * BLOCK_BYTES[fmt]), np.uint8)
    _load().synth_random_blocks(seed, fmt, N * (K // 256), emin, emax, int(allow_negative),
                                _ptr(out))
    return out


# ----------------------------------------------------------------------------------------
# Workload recipes.  Seeds: weights 1000*config + 10*tensor + 1, activations +2,
# outlier masks +3.  Weights are N(0, 0.02^2) floats packed to blocks.
# ----------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Gemm:
    name: str
    M: int
    K: int
    N: int
    fmt: int
    act: str          # "normal_outlier_f32", "normal_bf16", "rmsnorm_bf16", "student_t4_bf16"
    config: int
    tensor: int
    x_tensor: int = -1   # >= 0: share the activation rows of that tensor index

    @property
    def w_seed(self) -> int:
        return 1000 * self.config + 10 * self.tensor + 1

    @property
    def x_seed(self) -> int:
        t = self.tensor if self.x_tensor < 0 else self.x_tensor
        return 1000 * self.config + 10 * t + 2

    @property
    def x_dtype(self) -> int:
        return F32 if self.act.endswith("_f32") else BF16

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def w_bytes(self) -> int:
        return self.N * self.K // 256 * BLOCK_BYTES[self.fmt]


def make_weights(g: Gemm) -> np.ndarray:
    return pack(g.fmt, normal(g.w_seed, (g.N, g.K), 0.0, 0.02))


def make_acts(g: Gemm, rows: int | None = None) -> np.ndarray:
    """Activation rows [M x K]: float32 for *_f32 recipes, bf16 bits (uint16) otherwise."""
    M = g.M if rows is None else rows
    if g.act == "normal_outlier_f32":
        x = normal(g.x_seed, (M, g.K))
        return add_outliers(x, g.x_seed + 1, 0.01, 8.0)
    if g.act == "normal_bf16":
        return to_bf16_bits(normal(g.x_seed, (M, g.K)))
    if g.act == "rmsnorm_bf16":
        return to_bf16_bits(rmsnorm_rows(normal(g.x_seed, (M, g.K))))
    if g.act == "student_t4_bf16":
        return to_bf16_bits(student_t4(g.x_seed, (M, g.K)))
    raise ValueError(g.act)


def _c(config, tensor, name, M, K, N, fmt, act, x_tensor=-1):
    return Gemm(name, M, K, N, fmt, act, config, tensor, x_tensor)


# config 1: tiny Q4_K GEMM
CONFIG1 = [_c(1, 0, "tiny", 64, 1024, 1024, Q4_K, "normal_outlier_f32")]
# config 2: small-model projection set at one 512-row ubatch (all Q4_K)
CONFIG2 = [
    _c(2, 0, "qkv_gate", 512, 1024, 4096, Q4_K, "normal_bf16"),
    _c(2, 1, "up_gate", 512, 1024, 7168, Q4_K, "normal_bf16", x_tensor=0),  # same hidden rows
    _c(2, 2, "down", 512, 3584, 1024, Q4_K, "normal_bf16"),
]
# config 3: mid-size prefill at M = 512 and 4096 (the M = 512 rows are the first 512
# rows of the M = 4096 input; weights do not depend on M)
CONFIG3 = [
    _c(3, t, f"{name}_M{M}", M, K, N, fmt, "rmsnorm_bf16")
    for M in (512, 4096)
    for t, (name, K, N, fmt) in enumerate((("gate_up", 2560, 9728, Q4_K),
                                           ("down", 9728, 2560, Q4_K),
                                           ("attn_out", 4096, 2560, Q6_K)))
]
# config 4: long-prompt chunk sweep, Q4_K gate/up and Q6_K down
CONFIG4 = [
    _c(4, t, f"{name}_M{M}", M, K, N, fmt, "student_t4_bf16")
    for M in (512, 2048, 8192)
    for t, (name, K, N, fmt) in enumerate((("gate_up", 4096, 24576, Q4_K),
                                           ("down", 12288, 4096, Q6_K)))
]
# config 5: LM head on the last token (M = 1, 8) and the M = 512 comparison
CONFIG5 = [_c(5, 0, f"lm_head_M{M}", M, 4096, 152064, Q6_K, "rmsnorm_bf16") for M in (1, 8, 512)]
CONFIGS = {1: CONFIG1, 2: CONFIG2, 3: CONFIG3, 4: CONFIG4, 5: CONFIG5}
