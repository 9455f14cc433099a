"""GPU parity of the fusions either side of the GEMM against the CPU oracle,
through the C ABI.

RMSNorm -> quantiser: codes, block scales and code sums bit-exact against the
oracle's RMSNorm (binary64 sum of squares, scale rounded once to fp32) fed to
the per-32 quantiser.  The kernel sums the squares in its own order; a row
whose scale another summation order could change (the oracle reports the
interval every order's scale lies in) must match the oracle at one end of it.

SwiGLU: h = bf16(silu(gate) * up).  Against the oracle's fp64 value from its
fp64 GEMM: the GEMM's own bound tau = 1e-3 * ||x_row|| * max|w| on gate and up
carried through silu (|silu'| < 1.1), plus the fp32 evaluation (under 2^-17
relative) and the one bfloat16 rounding (2^-8 relative).  The fused kernel must also agree bit for
bit with the plain GEMM followed by the SwiGLU kernel (the same fp32 values
in the same order, the same SwiGLU arithmetic).
"""
import numpy as np
import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import oracle  # noqa: E402
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, bound, max_abs_w, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

# one bfloat16 rounding (2^-8 relative) plus the kernel's fp32 evaluation on the
# hardware exp2 and reciprocal (at most |g| * 2^-24 + 2^-20 < 2^-17 relative for
# |g| < 88.7)
BF16_REL = 2.0 ** -8 + 2.0 ** -16
# For g below -87.34 the reciprocal of 1 + e^-g falls below the fp32 normal
# range and the hardware reciprocal returns 0 (below -88.72 e^-g itself
# overflows), so silu(g) evaluates to -0 where the exact value is below
# 87.34 * e^-87.34 < 1.1e-36 in magnitude.
SILU_FLOOR = 1.1e-36


def _bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _residual_rows(seed: int, M: int, K: int) -> np.ndarray:
    """Pre-norm rows: heavy-tailed (Student t, 4 dof) with a few large outliers,
    plus rows of very different scales."""
    x = synth.student_t4(seed, (M, K))
    x = synth.add_outliers(x, seed + 1, 0.002, 30.0)
    x[1::5] *= np.float32(2.0 ** -12)
    x[2::7] *= np.float32(64.0)
    return x.astype(np.float32)


def _norm_weight(seed: int, K: int) -> np.ndarray:
    return synth.normal(seed, (K,), 1.0, 0.25).astype(np.float32)


def gpu_rms_hook(x: np.ndarray, g: np.ndarray, eps: float):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    d = torch.empty((M, K // 32), dtype=torch.float32, device=DEV)
    S = torch.empty((M, K // 32), dtype=torch.int32, device=DEV)
    qg.qgemm_rmsnorm_quantize_act(to_dev(x), to_dev(g), eps, M, K, q, d, S)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy(), S.cpu().numpy()


def check_rms_codes(x, g, eps, what=""):
    q, d, S = gpu_rms_hook(x, g, eps)
    oq, od, oS, amb, alt = oracle.rmsnorm_quantize(x, g, eps)
    for i in range(x.shape[0]):
        cands = [(oq, od, oS)] + (alt if amb[i] else [])
        ok = any(np.array_equal(q[i], cq[i]) and np.array_equal(d[i].view(np.uint32), cd[i].view(np.uint32))
                 and np.array_equal(S[i], cS[i]) for cq, cd, cS in cands)
        assert ok, f"{what}: row {i} differs (ambiguous scale: {bool(amb[i])})"
    return int(amb.sum())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [256, 1024, 2560, 4096, 12288, 20480])
def test_rmsnorm_quantize_bitexact(K, dtype):
    """Every register-chunk count of the kernel (K up to 2048, 4096, 8192, 16384,
    32768 per row) and both input types."""
    M = 23
    x = _residual_rows(1100 + K, M, K)
    x[0] = 0.0                                          # a zero row: r = 1/sqrt(eps), all codes 0
    x[3, :] = np.float32(-0.75)                         # a constant row
    x[4, 1:] = 0.0                                      # a single nonzero value
    g = _norm_weight(1101 + K, K)
    g[5] = 0.0                                          # a zeroed weight
    if dtype == "bf16":
        x = synth.to_bf16_bits(x)
    check_rms_codes(x, g, 1e-6, f"K={K} {dtype}")


def test_rmsnorm_order_sensitive_row():
    """The row whose scale depends on the summation order (small squares first
    give r = 1, the big value first gives 1 + 2^-23): either end is accepted."""
    K = 4096
    x = np.zeros((2, K), np.float32)
    x[:, :1000] = np.float32(1.5 * 2.0 ** -22)
    x[:, K - 1] = np.float32(64.0 * (1.0 - 2.0 ** -24))
    x[1] = x[1, ::-1]
    g = np.ones(K, np.float32)
    _, _, _, amb, _ = oracle.rmsnorm_quantize(x, g, 0.0)
    assert amb.all()
    check_rms_codes(x, g, 0.0, "order-sensitive rows")


def test_rmsnorm_eps_and_scale():
    M, K = 9, 1024
    x = _residual_rows(1110, M, K) * np.float32(1e-4)
    g = _norm_weight(1111, K)
    for eps in (0.0, 1e-6, 1e-2, 10.0):
        check_rms_codes(x, g, eps, f"eps={eps}")


@pytest.mark.parametrize("M,N,K", [(600, 4100, 1024), (130, 1000, 2560), (3, 333, 4096)])
def test_rmsnorm_workspace_then_gemm(M, N, K):
    """RMSNorm -> workspace -> GEMM (tiled and skinny) against the oracle GEMM
    of the oracle's normalised rows."""
    x = synth.to_bf16_bits(_residual_rows(1120 + M, M, K))
    g = _norm_weight(1121, K)
    eps = 1e-6
    W = synth.pack(qg.QG_Q4_K, synth.normal(1122 + N, (N, K), 0.0, 0.02))
    ws = torch.empty(qg.qgemm_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    qg.qgemm_rmsnorm_quantize_workspace(to_dev(x), to_dev(g), eps, M, K, ws)
    qg.qgemm_gemm_quantized(to_dev(W), qg.QG_Q4_K, ws, M, N, K, y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    r, lo, hi = oracle.rms_scale(x, eps)
    xn = oracle.rmsnorm(x, g, r)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 12)]))
    rows = rows[lo[rows] == hi[rows]]                   # scale fixed by every summation order
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(N - 33, N), rng.integers(0, N, 24)]))
    ref = oracle.gemm(qg.QG_Q4_K, W, xn, N, rows=rows, cols=cols)
    tol = bound(xn, rows, max_abs_w(qg.QG_Q4_K, W, N, K))
    err = np.abs(y[np.ix_(rows, cols)].astype(np.float64) - ref)
    assert np.all(err <= tol), float(np.max(err / tol))


@pytest.mark.parametrize("M,F", [(7, 64), (33, 4097), (512, 3584)])
def test_swiglu_kernel(M, F):
    """The SwiGLU kernel alone (vector and scalar column paths) on fp32 inputs,
    limits included."""
    y = synth.normal(1130 + F, (M, 2 * F), 0.0, 4.0)
    y[0, :6] = [0.0, -0.0, -100.0, 100.0, 88.5, -88.5]
    y[0, F:F + 6] = [3.0, 3.0, 2.0, 2.0, -1.0, 1.0]
    y[1, :F] = synth.normal(1131, (F,), 0.0, 30.0)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    qg.qgemm_swiglu(to_dev(y), M, F, h)
    torch.cuda.synchronize()
    got = _bf16_to_f64(h.cpu().view(torch.int16).numpy())
    ref = oracle.swiglu(y[:, :F].astype(np.float64), y[:, F:].astype(np.float64))
    assert np.all(np.abs(got - ref) <= BF16_REL * np.abs(ref) + SILU_FLOOR * np.abs(y[:, F:]) + 1e-38)
    assert got[0, 0] == 0.0 and got[0, 1] == 0.0 and got[0, 2] == 0.0 and got[0, 3] == 200.0


def gpu_swiglu(W, fmt, x, F):
    M, K = x.shape
    ws = torch.empty(qg.qgemm_swiglu_workspace_bytes(fmt, M, F, K), dtype=torch.uint8, device=DEV)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    qg.qgemm_prefill_swiglu(to_dev(W), fmt, to_dev(x), M, F, K, h, ws)
    torch.cuda.synchronize()
    return h.cpu().view(torch.int16).numpy().view(np.uint16)


def check_swiglu(h_bits, W, fmt, x, F, rows, cols, what):
    K = x.shape[1]
    got = _bf16_to_f64(h_bits[np.ix_(rows, cols)])
    href, gref, uref = oracle.gemm_swiglu(fmt, W, x, F, rows=rows, cols=cols)
    tau = bound(x, rows, max_abs_w(fmt, W, 2 * F, K))
    silu = np.abs(oracle.swiglu(gref, np.ones_like(gref)))
    pre = 1.1 * tau * (np.abs(uref) + tau) + silu * tau
    tol = pre + BF16_REL * (np.abs(href) + pre) + SILU_FLOOR * (np.abs(uref) + tau) + 1e-38
    err = np.abs(got - href)
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= tol), f"{what}: max err/tol {float(np.max(err / tol)):.3g}"


# shapes selecting every kernel the SwiGLU entry points dispatch
SW_SHAPES = [(qg.QG_Q4_K, 512, 3584, 1024),     # fused, 64x128 blocks
             (qg.QG_Q4_K, 500, 10250, 768),     # fused, one round of 128x256 then 64x256 blocks (ragged)
             (qg.QG_Q4_K, 2100, 5000, 512),     # fused, 128x256 blocks (ragged M and F)
             (qg.QG_Q4_K, 200, 3000, 1024),     # fused, 64x128 blocks with two K-groups
             (qg.QG_Q4_K, 100, 2100, 2048),     # fused, 32x64 blocks with four K-groups
             (qg.QG_Q4_K, 64, 512, 1024),       # small-grid GEMM + SwiGLU kernel
             (qg.QG_Q4_K, 3, 1000, 1024),       # skinny GEMM + SwiGLU kernel
             (qg.QG_Q6_K, 300, 700, 768),       # Q6_K GEMM + SwiGLU kernel
             (qg.QG_Q5_K, 300, 700, 768),       # Q5_K small-grid GEMM + SwiGLU kernel
             (qg.QG_Q5_K, 2, 500, 1024),        # Q5_K skinny GEMM + SwiGLU kernel
             (qg.QG_Q5_K, 512, 3584, 1024),     # Q5_K fused, 64x128 blocks
             (qg.QG_Q5_K, 200, 3000, 1024),     # Q5_K fused, 32x64 blocks with three K-groups
             (qg.QG_Q8_0, 512, 3584, 1024),     # Q8_0 fused, 64x128 blocks
             (qg.QG_Q8_0, 300, 700, 768),       # Q8_0 fused, 32x64 blocks with three K-groups
             (qg.QG_Q8_0, 70, 900, 512),        # Q8_0 fused, 32x64 blocks, one K-group (ragged F)
             (qg.QG_Q8_0, 6, 500, 1024)]        # Q8_0 skinny GEMM + SwiGLU kernel


@pytest.mark.parametrize("fmt,M,F,K", SW_SHAPES)
def test_gemm_swiglu_parity(fmt, M, F, K):
    name = qg.qgemm_kernel_name_swiglu(fmt, M, F, K)
    W = synth.pack(fmt, synth.normal(1140 + F, (2 * F, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(1141 + M, (M, K)))
    h = gpu_swiglu(W, fmt, x, F)
    if M * F <= 200 * 1000:
        rows, cols = np.arange(M), np.arange(F)
    else:
        rng = np.random.default_rng(M + F)
        rows = np.unique(np.concatenate([[0, M - 1], np.arange(M - 20, M), rng.integers(0, M, 16)]))
        cols = np.unique(np.concatenate([[0, F - 1], np.arange(F - 40, F), rng.integers(0, F, 30)]))
    check_swiglu(h, W, fmt, x, F, rows, cols, f"{M}x{F}x{K} fmt {fmt} ({name})")


@pytest.mark.parametrize("fmt,M,F,K", [(qg.QG_Q4_K, 512, 3584, 1024), (qg.QG_Q4_K, 2100, 5000, 512),
                                       (qg.QG_Q4_K, 500, 10250, 768),
                                       (qg.QG_Q4_K, 200, 3000, 1024), (qg.QG_Q4_K, 100, 2100, 2048),
                                       (qg.QG_Q5_K, 512, 3584, 1024), (qg.QG_Q5_K, 200, 3000, 1024),
                                       (qg.QG_Q8_0, 512, 3584, 1024), (qg.QG_Q8_0, 300, 700, 768),
                                       (qg.QG_Q8_0, 70, 900, 512)])
def test_fused_equals_gemm_then_swiglu(fmt, M, F, K):
    """The fused kernel's h is bit-identical to the plain GEMM's fp32 output fed
    to the SwiGLU kernel."""
    assert "_swiglu_" in qg.qgemm_kernel_name_swiglu(fmt, M, F, K)
    W = synth.pack(fmt, synth.normal(1150 + F, (2 * F, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(1151 + M, (M, K)))
    h = gpu_swiglu(W, fmt, x, F)
    ws = torch.empty(qg.qgemm_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, 2 * F), dtype=torch.float32, device=DEV)
    h2 = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    qg.qgemm_prefill(to_dev(W), fmt, to_dev(x), M, 2 * F, K, y, ws)
    qg.qgemm_swiglu(y, M, F, h2)
    torch.cuda.synchronize()
    assert np.array_equal(h, h2.cpu().view(torch.int16).numpy().view(np.uint16))


def test_rmsnorm_then_swiglu_pipeline():
    """RMSNorm -> quantiser -> fused gate+up SwiGLU from one workspace, against
    the oracle's normalised rows through its GEMM and SwiGLU."""
    M, F, K = 300, 2000, 1024
    x = synth.to_bf16_bits(_residual_rows(1160, M, K))
    g = _norm_weight(1161, K)
    W = synth.pack(qg.QG_Q4_K, synth.normal(1162, (2 * F, K), 0.0, 0.02))
    ws = torch.empty(qg.qgemm_swiglu_workspace_bytes(qg.QG_Q4_K, M, F, K), dtype=torch.uint8, device=DEV)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    qg.qgemm_rmsnorm_quantize_workspace(to_dev(x), to_dev(g), 1e-6, M, K, ws)
    qg.qgemm_gemm_quantized_swiglu(to_dev(W), qg.QG_Q4_K, ws, M, F, K, h)
    torch.cuda.synchronize()
    r, lo, hi = oracle.rms_scale(x, 1e-6)
    xn = oracle.rmsnorm(x, g, r)
    rng = np.random.default_rng(1163)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 12)]))
    rows = rows[lo[rows] == hi[rows]]
    cols = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, 30)]))
    check_swiglu(h.cpu().view(torch.int16).numpy().view(np.uint16), W, qg.QG_Q4_K, xn, F, rows, cols,
                 "rmsnorm -> swiglu")


@pytest.mark.parametrize("cfg,name", [(2, "up_gate"), (3, "gate_up_M512"), (4, "gate_up_M512"),
                                      (4, "gate_up_M2048")])
def test_gemm_swiglu_workload_sampled(cfg, name):
    """The workloads' gate+up projections (their 2F weight rows read as the
    stacked gate and up tensors) through the fused kernel."""
    gm = next(g for g in synth.CONFIGS[cfg] if g.name == name)
    F = gm.N // 2
    W, x = synth.make_weights(gm), synth.make_acts(gm)
    assert qg.qgemm_kernel_name_swiglu(gm.fmt, gm.M, F, gm.K).startswith("gemm_q4k_swiglu_")
    h = gpu_swiglu(W, gm.fmt, x, F)
    rng = np.random.default_rng(1170 + cfg)
    rows = np.unique(np.concatenate([[0, gm.M - 1], rng.integers(0, gm.M, 12)]))
    cols = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, 24)]))
    check_swiglu(h, W, gm.fmt, x, F, rows, cols, f"c{cfg} {name}")
