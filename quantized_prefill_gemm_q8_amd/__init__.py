"""Python binding of libqgemm.so (include/qgemm.h): the MI355X batched prefill
matmul over GGUF Q4_K / Q5_K / Q6_K / Q8_0 weights with int8-quantised activations.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libqgemm.so; this module turns torch tensors into device pointers
and the current HIP stream into a handle, and turns negative return codes into
exceptions.  There is no CPU path: if the library is missing, or the tensors
are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB as _LIB_PATH
from . import _build

QG_Q4_K, QG_Q6_K, QG_Q5_K, QG_Q8_0 = 0, 1, 2, 3
QG_F32, QG_BF16 = 0, 1
QG_PATH_AUTO, QG_PATH_TILED, QG_PATH_SKINNY = 0, 1, 2
QG_SKINNY_MAX_M = 8
QG_NOALLOC_SCRATCH_BYTES = 16 << 20
QG_ENOSCRATCH = -8
QG_PLANT_QUANTIZE = 1
QG_PLANT_MAX_SLEEPS = 1000000
BLOCK_BYTES = {QG_Q4_K: 144, QG_Q6_K: 210, QG_Q5_K: 176, QG_Q8_0: 272}  # per 256 values
SYMBOLS = ("qgemm_workspace_bytes", "qgemm_prefill", "qgemm_prefill_ex", "qgemm_lm_head",
           "qgemm_quantize_workspace", "qgemm_gemm_quantized",
           "qgemm_strerror", "qgemm_kernel_name", "qgemm_quantize_act", "qgemm_dequant",
           "qgemm_block_partials", "qgemm_deq_f16_workspace_bytes", "qgemm_prefill_deq_f16",
           "qgemm_deq_f16_kernel_name", "qgemm_to_f16", "qgemm_dequant_f16",
           "qgemm_quantize_workspace_a256", "qgemm_gemm_quantized_a256", "qgemm_prefill_a256",
           "qgemm_kernel_name_a256", "qgemm_quantize_act_a256",
           "qgemm_rmsnorm_quantize_workspace", "qgemm_rmsnorm_quantize_act",
           "qgemm_swiglu_workspace_bytes", "qgemm_gemm_quantized_swiglu", "qgemm_prefill_swiglu",
           "qgemm_kernel_name_swiglu", "qgemm_swiglu", "qgemm_sclk_probe", "qgemm_read_probe",
           "qgemm_prefill_noalloc", "qgemm_test_plant_delay")


class QgemmError(RuntimeError):
    def __init__(self, code: int, fn: str):
        super().__init__(f"{fn}: {qgemm_strerror(code)} (code {code})")
        self.code = code


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libqgemm.so (raises if it has not been built, or was built from other
    sources than the ones in the tree)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        if _build.is_stale():
            raise ImportError(f"{_LIB_PATH} was built from other sources than csrc/ and include/ "
                              "hold now: rebuild it (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.qgemm_workspace_bytes.argtypes = [i64, i64]
        lib.qgemm_workspace_bytes.restype = sz
        lib.qgemm_prefill.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp, sz, vp]
        lib.qgemm_prefill.restype = ci
        lib.qgemm_prefill_ex.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp, sz, vp, ci]
        lib.qgemm_prefill_ex.restype = ci
        lib.qgemm_lm_head.argtypes = [vp, ci, vp, ci, i64, i64, vp, vp, sz, vp]
        lib.qgemm_lm_head.restype = ci
        lib.qgemm_quantize_workspace.argtypes = [vp, ci, i64, i64, vp, sz, vp]
        lib.qgemm_quantize_workspace.restype = ci
        lib.qgemm_gemm_quantized.argtypes = [vp, ci, vp, sz, i64, i64, i64, vp, vp, ci]
        lib.qgemm_gemm_quantized.restype = ci
        lib.qgemm_kernel_name.argtypes = [ci, i64, i64, i64, ci]
        lib.qgemm_kernel_name.restype = ctypes.c_char_p
        lib.qgemm_strerror.argtypes = [ci]
        lib.qgemm_strerror.restype = ctypes.c_char_p
        lib.qgemm_quantize_act.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp]
        lib.qgemm_quantize_act.restype = ci
        lib.qgemm_dequant.argtypes = [vp, ci, i64, i64, vp, vp]
        lib.qgemm_dequant.restype = ci
        lib.qgemm_block_partials.argtypes = [vp, ci, vp, i64, i64, i64, vp, vp]
        lib.qgemm_block_partials.restype = ci
        lib.qgemm_deq_f16_workspace_bytes.argtypes = [i64, i64]
        lib.qgemm_deq_f16_workspace_bytes.restype = sz
        lib.qgemm_prefill_deq_f16.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp, sz, vp]
        lib.qgemm_prefill_deq_f16.restype = ci
        lib.qgemm_deq_f16_kernel_name.argtypes = [ci, i64, i64, i64]
        lib.qgemm_deq_f16_kernel_name.restype = ctypes.c_char_p
        lib.qgemm_to_f16.argtypes = [vp, ci, i64, i64, vp, vp]
        lib.qgemm_to_f16.restype = ci
        lib.qgemm_dequant_f16.argtypes = [vp, ci, i64, i64, vp, vp]
        lib.qgemm_dequant_f16.restype = ci
        lib.qgemm_quantize_workspace_a256.argtypes = [vp, ci, i64, i64, vp, sz, vp]
        lib.qgemm_quantize_workspace_a256.restype = ci
        lib.qgemm_gemm_quantized_a256.argtypes = [vp, ci, vp, sz, i64, i64, i64, vp, vp]
        lib.qgemm_gemm_quantized_a256.restype = ci
        lib.qgemm_prefill_a256.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp, sz, vp]
        lib.qgemm_prefill_a256.restype = ci
        lib.qgemm_kernel_name_a256.argtypes = [ci, i64, i64, i64]
        lib.qgemm_kernel_name_a256.restype = ctypes.c_char_p
        lib.qgemm_quantize_act_a256.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp]
        lib.qgemm_quantize_act_a256.restype = ci
        f32 = ctypes.c_float
        lib.qgemm_rmsnorm_quantize_workspace.argtypes = [vp, ci, vp, f32, i64, i64, vp, sz, vp]
        lib.qgemm_rmsnorm_quantize_workspace.restype = ci
        lib.qgemm_rmsnorm_quantize_act.argtypes = [vp, ci, vp, f32, i64, i64, vp, vp, vp, vp]
        lib.qgemm_rmsnorm_quantize_act.restype = ci
        lib.qgemm_swiglu_workspace_bytes.argtypes = [ci, i64, i64, i64]
        lib.qgemm_swiglu_workspace_bytes.restype = sz
        lib.qgemm_gemm_quantized_swiglu.argtypes = [vp, ci, vp, sz, i64, i64, i64, vp, vp]
        lib.qgemm_gemm_quantized_swiglu.restype = ci
        lib.qgemm_prefill_swiglu.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp, sz, vp]
        lib.qgemm_prefill_swiglu.restype = ci
        lib.qgemm_kernel_name_swiglu.argtypes = [ci, i64, i64, i64]
        lib.qgemm_kernel_name_swiglu.restype = ctypes.c_char_p
        lib.qgemm_swiglu.argtypes = [vp, i64, i64, vp, vp]
        lib.qgemm_swiglu.restype = ci
        lib.qgemm_sclk_probe.argtypes = [vp, ci, vp]
        lib.qgemm_sclk_probe.restype = ci
        lib.qgemm_read_probe.argtypes = [vp, i64, vp]
        lib.qgemm_read_probe.restype = ci
        lib.qgemm_prefill_noalloc.argtypes = [vp, ci, vp, ci, i64, i64, i64, vp, vp]
        lib.qgemm_prefill_noalloc.restype = ci
        lib.qgemm_test_plant_delay.argtypes = [ci, ci]
        lib.qgemm_test_plant_delay.restype = ci
        _lib = lib
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libqgemm takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libqgemm takes contiguous tensors only")
    return t.data_ptr()


def _dtype_code(x) -> int:
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.float32:
            return QG_F32
        if x.dtype == torch.bfloat16:
            return QG_BF16
        raise TypeError("activations must be torch.float32 or torch.bfloat16")
    raise TypeError("activations must be a torch tensor")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def _check(code: int, fn: str) -> None:
    if code != 0:
        raise QgemmError(code, fn)


def qgemm_strerror(code: int) -> str:
    return load().qgemm_strerror(code).decode()


def qgemm_kernel_name(fmt: int, M: int, N: int, K: int, path: int = QG_PATH_AUTO) -> str | None:
    r = load().qgemm_kernel_name(fmt, M, N, K, path)
    return None if r is None else r.decode()


def qgemm_workspace_bytes(M: int, K: int) -> int:
    return int(load().qgemm_workspace_bytes(M, K))


def qgemm_prefill(q_weights, fmt, x, M, N, K, y, workspace, stream=None, path=QG_PATH_AUTO):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_prefill_ex(_ptr(q_weights), fmt, _ptr(x), _dtype_code(x), M, N, K,
                                   _ptr(y), _ptr(workspace), ws_bytes, _stream(stream), path),
           "qgemm_prefill")


def qgemm_lm_head(q_weights, fmt, x_row, N, K, y, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_lm_head(_ptr(q_weights), fmt, _ptr(x_row), _dtype_code(x_row), N, K,
                                _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "qgemm_lm_head")


def qgemm_quantize_workspace(x, M, K, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_quantize_workspace(_ptr(x), _dtype_code(x), M, K, _ptr(workspace),
                                           ws_bytes, _stream(stream)), "qgemm_quantize_workspace")


def qgemm_gemm_quantized(q_weights, fmt, workspace, M, N, K, y, stream=None, path=QG_PATH_AUTO):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_gemm_quantized(_ptr(q_weights), fmt, _ptr(workspace), ws_bytes, M, N, K,
                                       _ptr(y), _stream(stream), path), "qgemm_gemm_quantized")


def qgemm_quantize_act(x, M, K, q, d, S, stream=None):
    _check(load().qgemm_quantize_act(_ptr(x), _dtype_code(x), M, K, _ptr(q), _ptr(d), _ptr(S),
                                     _stream(stream)), "qgemm_quantize_act")


def qgemm_dequant(q_weights, fmt, N, K, w, stream=None):
    _check(load().qgemm_dequant(_ptr(q_weights), fmt, N, K, _ptr(w), _stream(stream)),
           "qgemm_dequant")


def qgemm_block_partials(q_weights, fmt, qx, M, N, K, out, stream=None):
    _check(load().qgemm_block_partials(_ptr(q_weights), fmt, _ptr(qx), M, N, K, _ptr(out),
                                       _stream(stream)), "qgemm_block_partials")


# ---- per-256 activation scales (Q4_K) ----

def qgemm_quantize_workspace_a256(x, M, K, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_quantize_workspace_a256(_ptr(x), _dtype_code(x), M, K, _ptr(workspace),
                                                ws_bytes, _stream(stream)),
           "qgemm_quantize_workspace_a256")


def qgemm_gemm_quantized_a256(q_weights, fmt, workspace, M, N, K, y, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_gemm_quantized_a256(_ptr(q_weights), fmt, _ptr(workspace), ws_bytes, M, N, K,
                                            _ptr(y), _stream(stream)), "qgemm_gemm_quantized_a256")


def qgemm_prefill_a256(q_weights, fmt, x, M, N, K, y, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_prefill_a256(_ptr(q_weights), fmt, _ptr(x), _dtype_code(x), M, N, K, _ptr(y),
                                     _ptr(workspace), ws_bytes, _stream(stream)), "qgemm_prefill_a256")


def qgemm_kernel_name_a256(fmt: int, M: int, N: int, K: int) -> str | None:
    r = load().qgemm_kernel_name_a256(fmt, M, N, K)
    return None if r is None else r.decode()


def qgemm_quantize_act_a256(x, M, K, q, d, S, stream=None):
    _check(load().qgemm_quantize_act_a256(_ptr(x), _dtype_code(x), M, K, _ptr(q), _ptr(d), _ptr(S),
                                          _stream(stream)), "qgemm_quantize_act_a256")


# ---- the dequantise-to-fp16 branch (measured beside the int8 method) ----

def qgemm_deq_f16_workspace_bytes(M: int, K: int) -> int:
    return int(load().qgemm_deq_f16_workspace_bytes(M, K))


def qgemm_prefill_deq_f16(q_weights, fmt, x, M, N, K, y, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_prefill_deq_f16(_ptr(q_weights), fmt, _ptr(x), _dtype_code(x), M, N, K,
                                        _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "qgemm_prefill_deq_f16")


def qgemm_deq_f16_kernel_name(fmt: int, M: int, N: int, K: int) -> str | None:
    r = load().qgemm_deq_f16_kernel_name(fmt, M, N, K)
    return None if r is None else r.decode()


def qgemm_to_f16(x, M, K, x16, stream=None):
    _check(load().qgemm_to_f16(_ptr(x), _dtype_code(x), M, K, _ptr(x16), _stream(stream)),
           "qgemm_to_f16")


def qgemm_dequant_f16(q_weights, fmt, N, K, w16, stream=None):
    _check(load().qgemm_dequant_f16(_ptr(q_weights), fmt, N, K, _ptr(w16), _stream(stream)),
           "qgemm_dequant_f16")


# ---- fusions either side of the GEMM: RMSNorm -> quantiser, SwiGLU epilogue ----

def qgemm_rmsnorm_quantize_workspace(x, g, eps, M, K, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_rmsnorm_quantize_workspace(_ptr(x), _dtype_code(x), _ptr(g), float(eps), M, K,
                                                   _ptr(workspace), ws_bytes, _stream(stream)),
           "qgemm_rmsnorm_quantize_workspace")


def qgemm_rmsnorm_quantize_act(x, g, eps, M, K, q, d, S, stream=None):
    _check(load().qgemm_rmsnorm_quantize_act(_ptr(x), _dtype_code(x), _ptr(g), float(eps), M, K, _ptr(q),
                                             _ptr(d), _ptr(S), _stream(stream)), "qgemm_rmsnorm_quantize_act")


def qgemm_swiglu_workspace_bytes(fmt: int, M: int, F: int, K: int) -> int:
    return int(load().qgemm_swiglu_workspace_bytes(fmt, M, F, K))


def qgemm_gemm_quantized_swiglu(q_weights, fmt, workspace, M, F, K, h, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_gemm_quantized_swiglu(_ptr(q_weights), fmt, _ptr(workspace), ws_bytes, M, F, K,
                                              _ptr(h), _stream(stream)), "qgemm_gemm_quantized_swiglu")


def qgemm_prefill_swiglu(q_weights, fmt, x, M, F, K, h, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qgemm_prefill_swiglu(_ptr(q_weights), fmt, _ptr(x), _dtype_code(x), M, F, K, _ptr(h),
                                       _ptr(workspace), ws_bytes, _stream(stream)), "qgemm_prefill_swiglu")


def qgemm_kernel_name_swiglu(fmt: int, M: int, F: int, K: int) -> str | None:
    r = load().qgemm_kernel_name_swiglu(fmt, M, F, K)
    return None if r is None else r.decode()


def qgemm_swiglu(y, M, F, h, stream=None):
    _check(load().qgemm_swiglu(_ptr(y), M, F, _ptr(h), _stream(stream)), "qgemm_swiglu")


# ---- no allocation (static scratch inside the library) ----

def qgemm_prefill_noalloc(q_weights, fmt, x, M, N, K, y, stream=None):
    _check(load().qgemm_prefill_noalloc(_ptr(q_weights), fmt, _ptr(x), _dtype_code(x), M, N, K, _ptr(y),
                                        _stream(stream)), "qgemm_prefill_noalloc")


# ---- diagnostics ----

def qgemm_sclk_probe(ticks, iters, stream=None):
    _check(load().qgemm_sclk_probe(_ptr(ticks), iters, _stream(stream)), "qgemm_sclk_probe")


def qgemm_read_probe(src, nbytes, stream=None):
    """Read nbytes of the device buffer src once (the floor of a bandwidth-bound launch)."""
    _check(load().qgemm_read_probe(_ptr(src), nbytes, _stream(stream)), "qgemm_read_probe")


def qgemm_test_plant_delay(kernel, sleeps):
    """Planted delay of one kernel, for the timing falsifier (0 removes it)."""
    _check(load().qgemm_test_plant_delay(kernel, sleeps), "qgemm_test_plant_delay")


def measure_sclk_mhz(iters: int = 8000, stream=None, device="cuda") -> float:
    """Shader clock (MHz) under int8 matrix-core load, from qgemm_sclk_probe."""
    ticks = torch.zeros(3, dtype=torch.int64, device=device)
    qgemm_sclk_probe(ticks, iters, stream)
    t = ticks.cpu().tolist()
    if t[1] <= 0:
        raise RuntimeError("clock probe: no reference ticks")
    return round(100.0 * t[0] / t[1], 1)


# ---- plumbing helpers: device buffers for callers that do not manage their own ----

def alloc_workspace(M: int, K: int, device="cuda") -> torch.Tensor:
    n = qgemm_workspace_bytes(M, K)
    if n == 0:
        raise QgemmError(-1, "qgemm_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(q_weights: torch.Tensor, fmt: int, x: torch.Tensor, N: int, path=QG_PATH_AUTO,
            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x . W^T for x [M, K] on the GPU; allocates y (and the workspace if not given)."""
    M, K = x.shape
    if workspace is None:
        workspace = alloc_workspace(M, K, x.device)
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    qgemm_prefill(q_weights, fmt, x, M, N, K, y, workspace, stream, path)
    return y
