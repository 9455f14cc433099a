"""CPU oracle for the Q4_K / Q6_K x int8 prefill GEMM -- TEST INFRASTRUCTURE.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never links, loads or calls it, and it
shares no code with the GPU library.  The arithmetic lives in ``oracle.c``
(plain C, fp64 combine, exact int32 partials); this module only marshals numpy
arrays into it.

Functions and the passage each follows are documented in ``oracle.c``.  Every
function here is pinned by CPU tests against closed forms, hand-packed blocks,
brute-force fp64 dequantise-then-matmul and a textbook integer matmul.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q4_K = 0
Q6_K = 1
Q5_K = 2
Q8_0 = 3
F32 = 0
BF16 = 1
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q5_K: 176, Q8_0: 272}   # bytes per 256 values (Q8_0: 8 x 34)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc: -O3, OpenMP, IEEE semantics (no fast-math, no contraction:
    the optimiser may not reassociate or fuse floating-point operations)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ci
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_decode_q4k.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_decode_q4k.restype = None
    lib.oracle_decode_q5k.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_decode_q5k.restype = None
    lib.oracle_decode_q80.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_decode_q80.restype = None
    lib.oracle_decode_q6k.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.oracle_decode_q6k.restype = None
    lib.oracle_dequant.argtypes = [ci, vp, i64, i64, vp]
    lib.oracle_dequant.restype = None
    lib.oracle_quantize_act.argtypes = [vp, ci, i64, i64, vp, vp, vp]
    lib.oracle_quantize_act.restype = None
    lib.oracle_block_partials.argtypes = [ci, vp, vp, i64, i64, i64, vp]
    lib.oracle_block_partials.restype = None
    lib.oracle_gemm.argtypes = [ci, vp, vp, ci, i64, i64, i64, vp, i64, vp, i64, vp]
    lib.oracle_gemm.restype = ci
    lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_x_to_f16.argtypes = [vp, ci, i64, i64, vp]
    lib.oracle_x_to_f16.restype = None
    lib.oracle_dequant_f16.argtypes = [ci, vp, i64, i64, vp]
    lib.oracle_dequant_f16.restype = None
    lib.oracle_gemm_deq_f16.argtypes = [ci, vp, vp, ci, i64, i64, i64, vp, i64, vp, i64, vp, vp]
    lib.oracle_gemm_deq_f16.restype = ci
    lib.oracle_quantize_act256.argtypes = [vp, ci, i64, i64, vp, vp, vp]
    lib.oracle_quantize_act256.restype = None
    lib.oracle_gemm_a256.argtypes = [vp, vp, ci, i64, i64, i64, vp, i64, vp, i64, vp]
    lib.oracle_gemm_a256.restype = ci
    lib.oracle_rms_scale.argtypes = [vp, ci, i64, i64, ctypes.c_float, vp, vp, vp]
    lib.oracle_rms_scale.restype = None
    lib.oracle_rmsnorm.argtypes = [vp, ci, vp, vp, i64, i64, vp]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_swiglu.argtypes = [vp, vp, i64, vp]
    lib.oracle_swiglu.restype = None
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _x_dtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("activations must be float32 or bf16 bit patterns (uint16)")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use (the CPU baseline's core count)."""
    return int(_load().oracle_num_threads())


def half_to_double(h: int) -> float:
    return float(_load().oracle_half_to_double(h))


def decode_q4k(W: np.ndarray, N: int, K: int):
    """Returns (q [N,K] uint8, sc [N,K/32], m [N,K/32] uint8, d [N,K/256], dmin [N,K/256] f64)."""
    W = np.ascontiguousarray(W, np.uint8)
    assert W.size == N * K // 256 * 144
    q = np.empty((N, K), np.uint8)
    sc = np.empty((N, K // 32), np.uint8)
    m = np.empty((N, K // 32), np.uint8)
    d = np.empty((N, K // 256), np.float64)
    dmin = np.empty((N, K // 256), np.float64)
    _load().oracle_decode_q4k(_p(W), N, K, _p(q), _p(sc), _p(m), _p(d), _p(dmin))
    return q, sc, m, d, dmin


def decode_q5k(W: np.ndarray, N: int, K: int):
    """Returns (q [N,K] uint8 in 0..31, sc [N,K/32], m [N,K/32] uint8, d, dmin [N,K/256] f64)."""
    W = np.ascontiguousarray(W, np.uint8)
    assert W.size == N * K // 256 * 176
    q = np.empty((N, K), np.uint8)
    sc = np.empty((N, K // 32), np.uint8)
    m = np.empty((N, K // 32), np.uint8)
    d = np.empty((N, K // 256), np.float64)
    dmin = np.empty((N, K // 256), np.float64)
    _load().oracle_decode_q5k(_p(W), N, K, _p(q), _p(sc), _p(m), _p(d), _p(dmin))
    return q, sc, m, d, dmin


def decode_q80(W: np.ndarray, N: int, K: int):
    """Q8_0 (K % 32 == 0): returns (q [N,K] int8, d [N,K/32] f64)."""
    W = np.ascontiguousarray(W, np.uint8)
    assert K % 32 == 0 and W.size == N * K // 32 * 34
    q = np.empty((N, K), np.int8)
    d = np.empty((N, K // 32), np.float64)
    _load().oracle_decode_q80(_p(W), N, K, _p(q), _p(d))
    return q, d


def decode_q6k(W: np.ndarray, N: int, K: int):
    """Returns (q6 [N,K] uint8 in 0..63, sc [N,K/16] int8, d [N,K/256] f64)."""
    W = np.ascontiguousarray(W, np.uint8)
    assert W.size == N * K // 256 * 210
    q = np.empty((N, K), np.uint8)
    sc = np.empty((N, K // 16), np.int8)
    d = np.empty((N, K // 256), np.float64)
    _load().oracle_decode_q6k(_p(W), N, K, _p(q), _p(sc), _p(d))
    return q, sc, d


def dequant(fmt: int, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Dequantised weights [N, K] in fp64."""
    W = np.ascontiguousarray(W, np.uint8)
    assert W.size == N * K // 256 * BLOCK_BYTES[fmt]
    w = np.empty((N, K), np.float64)
    _load().oracle_dequant(fmt, _p(W), N, K, _p(w))
    return w


def quantize_act(x: np.ndarray):
    """x [M, K] float32 or bf16 bits -> (q int8 [M,K], d float32 [M,K/32], S int32 [M,K/32])."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 32 == 0
    q = np.empty((M, K), np.int8)
    d = np.empty((M, K // 32), np.float32)
    S = np.empty((M, K // 32), np.int32)
    _load().oracle_quantize_act(_p(x), _x_dtype(x), M, K, _p(q), _p(d), _p(S))
    return q, d, S


def block_partials(fmt: int, W: np.ndarray, qx: np.ndarray, N: int) -> np.ndarray:
    """Integer partials: Q4_K, Q5_K, Q8_0 [M, N, K/32], Q6_K [M, N, K/16] (int32)."""
    W = np.ascontiguousarray(W, np.uint8)
    qx = np.ascontiguousarray(qx, np.int8)
    M, K = qx.shape
    assert W.size == N * K // 256 * BLOCK_BYTES[fmt]
    L = 16 if fmt == Q6_K else 32
    out = np.empty((M, N, K // L), np.int32)
    _load().oracle_block_partials(fmt, _p(W), _p(qx), M, N, K, _p(out))
    return out


def gemm(fmt: int, W: np.ndarray, x: np.ndarray, N: int, rows=None, cols=None) -> np.ndarray:
    """y [len(rows), len(cols)] in fp64 (all rows / columns when None)."""
    W = np.ascontiguousarray(W, np.uint8)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 256 == 0 and W.size == N * K // 256 * BLOCK_BYTES[fmt]
    r = None if rows is None else np.ascontiguousarray(rows, np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, np.int64)
    if r is not None:
        assert r.size == 0 or (r.min() >= 0 and r.max() < M)
    if c is not None:
        assert c.size == 0 or (c.min() >= 0 and c.max() < N)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    y = np.empty((nr, nc), np.float64)
    if nr == 0 or nc == 0:
        return y
    rc = _load().oracle_gemm(fmt, _p(W), _p(x), _x_dtype(x), M, N, K,
                             None if r is None else _p(r), nr,
                             None if c is None else _p(c), nc, _p(y))
    if rc != 0:
        raise MemoryError("oracle_gemm: allocation failed")
    return y


def f64_to_f16(v: float) -> int:
    """binary16 bits of the value nearest to v (ties to even)."""
    return int(_load().oracle_f64_to_f16(float(v)))


def x_to_f16(x: np.ndarray) -> np.ndarray:
    """x [M, K] float32 or bf16 bits -> binary16 bits [M, K] (uint16)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    out = np.empty((M, K), np.uint16)
    _load().oracle_x_to_f16(_p(x), _x_dtype(x), M, K, _p(out))
    return out


def dequant_f16(fmt: int, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """binary16 weights [N, K] (uint16 bits) of the dequantise-to-fp16 branch."""
    W = np.ascontiguousarray(W, np.uint8)
    assert W.size == N * K // 256 * BLOCK_BYTES[fmt]
    out = np.empty((N, K), np.uint16)
    _load().oracle_dequant_f16(fmt, _p(W), N, K, _p(out))
    return out


def gemm_deq_f16(fmt: int, W: np.ndarray, x: np.ndarray, N: int, rows=None, cols=None):
    """(y, yabs) [len(rows), len(cols)] in fp64 for the dequantise-to-fp16 branch:
    y = x16 . w16^T and yabs = sum_k |x16 * w16|."""
    W = np.ascontiguousarray(W, np.uint8)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 256 == 0 and W.size == N * K // 256 * BLOCK_BYTES[fmt]
    r = None if rows is None else np.ascontiguousarray(rows, np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    y = np.empty((nr, nc), np.float64)
    ya = np.empty((nr, nc), np.float64)
    if nr == 0 or nc == 0:
        return y, ya
    rc = _load().oracle_gemm_deq_f16(fmt, _p(W), _p(x), _x_dtype(x), M, N, K,
                                     None if r is None else _p(r), nr,
                                     None if c is None else _p(c), nc, _p(y), _p(ya))
    if rc != 0:
        raise MemoryError("oracle_gemm_deq_f16: allocation failed")
    return y, ya


def quantize_act256(x: np.ndarray):
    """Per-256 activation blocks: x [M, K] -> (q int8 [M,K], d float32 [M,K/256],
    S int32 [M,K/32] per 32-value sub-block)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 256 == 0
    q = np.empty((M, K), np.int8)
    d = np.empty((M, K // 256), np.float32)
    S = np.empty((M, K // 32), np.int32)
    _load().oracle_quantize_act256(_p(x), _x_dtype(x), M, K, _p(q), _p(d), _p(S))
    return q, d, S


def gemm_a256(W: np.ndarray, x: np.ndarray, N: int, rows=None, cols=None) -> np.ndarray:
    """Q4_K GEMM with per-256 activation scales: y [len(rows), len(cols)] in fp64."""
    W = np.ascontiguousarray(W, np.uint8)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 256 == 0 and W.size == N * K // 256 * BLOCK_BYTES[Q4_K]
    r = None if rows is None else np.ascontiguousarray(rows, np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    y = np.empty((nr, nc), np.float64)
    if nr == 0 or nc == 0:
        return y
    rc = _load().oracle_gemm_a256(_p(W), _p(x), _x_dtype(x), M, N, K,
                                  None if r is None else _p(r), nr,
                                  None if c is None else _p(c), nc, _p(y))
    if rc != 0:
        raise MemoryError("oracle_gemm_a256: allocation failed")
    return y


def rms_scale(x: np.ndarray, eps: float):
    """RMSNorm scale per row: (r32, r32_lo, r32_hi), float32 [M] each.  r32 is the
    oracle's own; [r32_lo, r32_hi] holds the r32 of any summation order of the
    row's sum of squares (equal ends: every order gives r32)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    r, lo, hi = (np.empty(M, np.float32) for _ in range(3))
    _load().oracle_rms_scale(_p(x), _x_dtype(x), M, K, float(np.float32(eps)), _p(r), _p(lo), _p(hi))
    return r, lo, hi


def rmsnorm(x: np.ndarray, g: np.ndarray, r32: np.ndarray) -> np.ndarray:
    """Normalised rows xn = f32(f32(x * r32[row]) * g[col]), float32 [M, K]."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    g = np.ascontiguousarray(g, np.float32)
    r32 = np.ascontiguousarray(r32, np.float32)
    assert g.shape == (K,) and r32.shape == (M,)
    xn = np.empty((M, K), np.float32)
    _load().oracle_rmsnorm(_p(x), _x_dtype(x), _p(g), _p(r32), M, K, _p(xn))
    return xn


def rmsnorm_quantize(x: np.ndarray, g: np.ndarray, eps: float):
    """RMSNorm then the per-32 quantiser: (q, d, S) as quantize_act returns them,
    plus the rows whose r32 another summation order could change (a bool mask)
    and, for those, the codes of the interval's two ends: alt = [(q, d, S) at
    r32_lo, (q, d, S) at r32_hi]."""
    r, lo, hi = rms_scale(x, eps)
    q, d, S = quantize_act(rmsnorm(x, g, r))
    amb = lo != hi
    alt = [quantize_act(rmsnorm(x, g, np.where(amb, e, r))) for e in (lo, hi)]
    return q, d, S, amb, alt


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up elementwise, in fp64."""
    gate = np.ascontiguousarray(gate, np.float64)
    up = np.ascontiguousarray(up, np.float64)
    assert gate.shape == up.shape
    h = np.empty(gate.shape, np.float64)
    _load().oracle_swiglu(_p(gate), _p(up), gate.size, _p(h))
    return h


def gemm_swiglu(fmt: int, W: np.ndarray, x: np.ndarray, F: int, rows=None, cols=None):
    """SwiGLU of a stacked gate+up projection (W holds 2F rows: gate, then up):
    h [len(rows), len(cols)] in fp64, cols indexing 0..F-1, and the gate and up
    GEMM outputs it was formed from."""
    M = x.shape[0]
    c = np.arange(F, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    y = gemm(fmt, W, x, 2 * F, rows=rows, cols=np.concatenate([c, c + F]))
    g, u = y[:, :c.size], y[:, c.size:]
    return swiglu(g, u), g, u


class Oracle:
    """The same functions bound to another build of oracle.c (used by the tests
    that plant a mistake in a copy of the source and check that a pin fails)."""

    def __init__(self, path: str):
        self._lib = _bind(path)

    def _call(self, fn, *a, **k):
        global _lib
        saved = _lib
        _lib = self._lib
        try:
            return fn(*a, **k)
        finally:
            _lib = saved

    def __getattr__(self, name):
        fn = globals()[name]
        return lambda *a, **k: self._call(fn, *a, **k)


def source_path() -> str:
    return _SRC
