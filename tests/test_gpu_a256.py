"""GPU parity of the per-256 activation-scale variant (Q4_K) against the CPU
oracle's per-256 functions, through the C ABI.

Bit-exact: the quantiser's codes, super-block scales and sub-block code sums.
GEMM output within the method's bound |dy| <= 1e-3 * ||x_row||_2 * max|w| on
every element at small sizes and on sampled elements at the workloads' sizes,
for every kernel the per-256 entry point dispatches (the three LDS block shapes
with the integer sub-block combine, the small-grid kernel and the skinny
kernel); exact on the textbook integer case.
"""
import numpy as np
import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import oracle  # noqa: E402
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, bound, check, max_abs_w, to_dev  # noqa: E402
import pins  # noqa: E402

pytestmark = pytest.mark.gpu


def gpu_a256(W: np.ndarray, x: np.ndarray, N: int) -> np.ndarray:
    M, K = x.shape
    ws = torch.empty(qg.qgemm_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    qg.qgemm_prefill_a256(to_dev(W), qg.QG_Q4_K, to_dev(x), M, N, K, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_a256_bitexact(dtype):
    M, K = 21, 1024
    x = synth.normal(801, (M, K))
    x[::4] *= np.float32(16.0)
    x[1, :256] = 0.0
    x[2, 256:512] = np.float32(2.0 ** -140)
    x[3, 512:768] = np.tile(np.float32([127, 0.5, 1.5, 2.5, -0.5, -2.5, 126.5, -3.5]), 32)
    x[4, 5] = np.float32(1e30)
    if dtype == "bf16":
        x = synth.to_bf16_bits(x)
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    d = torch.empty((M, K // 256), dtype=torch.float32, device=DEV)
    S = torch.empty((M, K // 32), dtype=torch.int32, device=DEV)
    qg.qgemm_quantize_act_a256(to_dev(x), M, K, q, d, S)
    torch.cuda.synchronize()
    oq, od, oS = oracle.quantize_act256(x)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), od.view(np.uint32))
    assert np.array_equal(S.cpu().numpy(), oS)


# shapes selecting each kernel of the per-256 dispatch (ragged tails included)
SHAPES = [(2100, 4100, 512),    # 64x128 blocks (long prompts)
          (600, 4200, 768),     # 64x128 blocks
          (600, 1700, 1024),    # 64x128 blocks, two K-groups
          (200, 2400, 2048),    # 32x64 blocks, four K-groups
          (64, 1024, 1024),     # small-grid kernel
          (3, 300, 1024)]       # skinny kernel


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_a256_parity(M, N, K):
    W = synth.pack(qg.QG_Q4_K, synth.normal(810 + M, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(811 + N, (M, K)))
    y = gpu_a256(W, x, N)
    if M * N <= 300 * 1000:
        rows, cols = np.arange(M), np.arange(N)
    else:
        rng = np.random.default_rng(M + N)
        rows = np.unique(np.concatenate([[0, M - 1], np.arange(M - 20, M), rng.integers(0, M, 16)]))
        cols = np.unique(np.concatenate([[0, N - 1], np.arange(N - 40, N), rng.integers(0, N, 30)]))
    ref = oracle.gemm_a256(W, x, N, rows=rows, cols=cols)
    tol = bound(x, rows, max_abs_w(qg.QG_Q4_K, W, N, K))
    check(y[np.ix_(rows, cols)], ref, tol, f"a256 {M}x{N}x{K} ({qg.qgemm_kernel_name_a256(0, M, N, K)})")


def test_gemm_a256_textbook_exact():
    M, N, K = 600, 1700, 1024         # the two-group 64x128 kernel
    W, wv = pins._textbook_blocks(qg.QG_Q4_K, N, K, seed=820)
    rng = np.random.default_rng(821)
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, ::256] = 127
    y = gpu_a256(W, xi.astype(np.float32), N)
    assert np.array_equal(y.astype(np.float64), (xi @ wv.T).astype(np.float64))


@pytest.mark.parametrize("cfg,name", [(2, "qkv_gate"), (3, "gate_up_M512"), (4, "gate_up_M512"),
                                      (4, "gate_up_M2048")])
def test_gemm_a256_workload_sampled(cfg, name):
    g = next(g for g in synth.CONFIGS[cfg] if g.name == name)
    W, x = synth.make_weights(g), synth.make_acts(g)
    y = gpu_a256(W, x, g.N)
    rng = np.random.default_rng(830 + cfg)
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.integers(0, g.M, 12)]))
    cols = np.unique(np.concatenate([[0, g.N - 1], rng.integers(0, g.N, 24)]))
    ref = oracle.gemm_a256(W, x, g.N, rows=rows, cols=cols)
    tol = bound(x, rows, max_abs_w(qg.QG_Q4_K, W, g.N, g.K))
    check(y[np.ix_(rows, cols)], ref, tol, f"a256 c{cfg} {name}")
