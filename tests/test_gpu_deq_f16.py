"""GPU parity of the dequantise-to-fp16 design branch (qgemm_prefill_deq_f16 and
its hooks) against the CPU oracle's fp16 functions.

Bit-exact: the binary16 activations, and the binary16 weights of the GEMM's own
decoder (a zero weight compares equal to either sign of zero).  GEMM output:
the products x16*w16 are exact in fp32, so the only difference from the
oracle's exact sum is the fp32 accumulation, bounded for any summation order by
|dy| <= K * 2^-24 / (1 - K * 2^-24) * sum_k |x16*w16| (gamma_K); checked on every
element at small sizes and on sampled elements at the workloads' sizes, plus the
exact textbook case (integer weights and activations: an integer matmul).
"""
import numpy as np
import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import oracle  # noqa: E402
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import pins  # noqa: E402

pytestmark = pytest.mark.gpu


def _plus_zero(bits: np.ndarray) -> np.ndarray:
    b = bits.copy()
    b[b == 0x8000] = 0
    return b


def gamma(K: int) -> float:
    u = 2.0 ** -24
    return K * u / (1 - K * u)


def gpu_deq(W: np.ndarray, x: np.ndarray, N: int, fmt: int = qg.QG_Q4_K) -> np.ndarray:
    M, K = x.shape
    ws = torch.empty(qg.qgemm_deq_f16_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    qg.qgemm_prefill_deq_f16(to_dev(W), fmt, to_dev(x), M, N, K, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_deq(y: np.ndarray, W, x, N, K, rows=None, cols=None, what="", fmt=qg.QG_Q4_K):
    ref, refabs = oracle.gemm_deq_f16(fmt, W, x, N, rows=rows, cols=cols)
    sub = y if rows is None else y[np.ix_(rows, cols)]
    err = np.abs(sub.astype(np.float64) - ref)
    tol = gamma(K) * refabs
    assert np.all(np.isfinite(sub)), what
    assert np.all(err <= tol), f"{what}: max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_to_f16_bitexact(dtype):
    M, K = 9, 512
    x = synth.normal(601, (M, K)) * np.float32(4.0)
    x[0, :10] = [0.0, -0.0, 1e-9, -7e-6, 65519.0, 65520.0, -1e6, 6e-5, 2.0 ** -24, 1.00048828125]
    if dtype == "bf16":
        x = synth.to_bf16_bits(x)
    x16 = torch.empty((M, K), dtype=torch.int16, device=DEV)
    qg.qgemm_to_f16(to_dev(x), M, K, x16)
    torch.cuda.synchronize()
    got = x16.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.x_to_f16(x))


@pytest.mark.parametrize("fmt", [qg.QG_Q4_K, qg.QG_Q6_K], ids=["q4k", "q6k"])
def test_dequant_f16_bitexact(fmt):
    N, K = 40, 1024
    Ws = [synth.random_blocks(fmt, N, K, seed=610 + fmt, emin=1, emax=23),
          synth.random_blocks(fmt, N, K, seed=620 + fmt, emin=8, emax=16),
          synth.pack(fmt, synth.normal(630 + fmt, (N, K), 0.0, 0.02))]
    for W in Ws:
        w16 = torch.empty((N, K), dtype=torch.int16, device=DEV)
        qg.qgemm_dequant_f16(to_dev(W), fmt, N, K, w16)
        torch.cuda.synchronize()
        got = w16.cpu().numpy().view(np.uint16)
        assert np.array_equal(_plus_zero(got), _plus_zero(oracle.dequant_f16(fmt, W, N, K)))


FMTS = [qg.QG_Q4_K, qg.QG_Q6_K]
FID = ["q4k", "q6k"]


@pytest.mark.parametrize("fmt", FMTS, ids=FID)
@pytest.mark.parametrize("M,N,K", [(64, 1024, 1024), (200, 300, 512), (130, 260, 768), (1, 77, 256),
                                   (129, 129, 256), (600, 500, 2560)])
def test_gemm_full_parity(M, N, K, fmt):
    W = synth.pack(fmt, synth.normal(640 + M, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(650 + N, (M, K)))
    check_deq(gpu_deq(W, x, N, fmt), W, x, N, K, what=f"{M}x{N}x{K}", fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FID)
@pytest.mark.parametrize("M,N,K", [(1100, 9000, 512), (700, 11000, 512), (300, 8500, 512),
                                   (520, 4000, 768), (520, 2560, 1280), (500, 2000, 768)])
def test_gemm_large_tiles_sampled(M, N, K, fmt):
    """The 256x256, 256x128 and 128x128 block kernels and the two-group 64x128
    and four-group 128x64 (Q4_K) K splits, on ragged shapes (tails in M and N)."""
    W = synth.pack(fmt, synth.normal(690 + M, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(691 + N, (M, K)))
    y = gpu_deq(W, x, N, fmt)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(M - 40, M), rng.integers(0, M, 24)]))
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(N - 70, N), rng.integers(0, N, 40)]))
    check_deq(y, W, x, N, K, rows=rows, cols=cols, what=f"{M}x{N}x{K}", fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FID)
def test_gemm_f32_input_and_wide_scales(fmt):
    M, N, K = 96, 160, 1024
    W = synth.random_blocks(fmt, N, K, seed=660 + fmt, emin=5, emax=18)
    x = synth.normal(661, (M, K)) * np.float32(3.0)
    check_deq(gpu_deq(W, x, N, fmt), W, x, N, K, what="f32 input, random blocks", fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FID)
def test_gemm_textbook_exact(fmt):
    M, N, K = 70, 130, 512
    W, wv = pins._textbook_blocks(fmt, N, K, seed=670 + fmt)
    xi = pins._integer_acts(M, K, seed=671)
    y = gpu_deq(W, xi.astype(np.float32), N, fmt)
    assert np.array_equal(y.astype(np.float64), (xi @ wv.T).astype(np.float64))


@pytest.mark.parametrize("cfg,name", [(2, "qkv_gate"), (2, "up_gate"), (2, "down"),
                                      (3, "gate_up_M512"), (3, "down_M512"), (3, "attn_out_M512"),
                                      (4, "gate_up_M512"), (4, "down_M512")])
def test_gemm_workload_sampled(cfg, name):
    g = next(g for g in synth.CONFIGS[cfg] if g.name == name)
    W, x = synth.make_weights(g), synth.make_acts(g)
    y = gpu_deq(W, x, g.N, g.fmt)
    rng = np.random.default_rng(680 + cfg)
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.integers(0, g.M, 14)]))
    cols = np.unique(np.concatenate([[0, g.N - 1], rng.integers(0, g.N, 30)]))
    check_deq(y, W, x, g.N, g.K, rows=rows, cols=cols, what=f"c{cfg} {name}", fmt=g.fmt)


def test_rejects_unknown_format():
    W = torch.zeros(210 * 4, dtype=torch.uint8, device=DEV)
    x = torch.zeros((2, 256), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((2, 4), dtype=torch.float32, device=DEV)
    ws = torch.empty(qg.qgemm_deq_f16_workspace_bytes(2, 256), dtype=torch.uint8, device=DEV)
    with pytest.raises(qg.QgemmError):
        qg.qgemm_prefill_deq_f16(W, 2, x, 2, 4, 256, y, ws)
