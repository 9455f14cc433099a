"""The library's calls under HIP graph capture: the quantiser and every GEMM
kernel family (tiled, K-split tiled, small-grid, skinny, LM head) captured on a
torch CUDA graph and replayed several times, with unrelated eager work and
synchronisations between the replays; every replay must reproduce the eager
result bit for bit (same kernels, same arguments), and the eager result is
checked against the CPU oracle."""
import numpy as np
import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import oracle  # noqa: E402
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, bound, check, max_abs_w, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

# (fmt, M, N, K): one shape per kernel family the dispatcher picks
CASES = [
    (qg.QG_Q4_K, 577, 8240, 768),     # 64x128 tiles
    (qg.QG_Q4_K, 170, 2800, 2816),    # 32x64 blocks, K split over 4 groups
    (qg.QG_Q4_K, 100, 200, 512),      # small grid, K split over waves
    (qg.QG_Q6_K, 300, 8300, 512),     # Q6_K 64x128 tiles
    (qg.QG_Q6_K, 5, 3000, 1024),      # skinny
]


def test_graph_replays_match_eager():
    stream = torch.cuda.Stream()
    prob = []
    for i, (fmt, M, N, K) in enumerate(CASES):
        W = synth.pack(fmt, synth.normal(700 + i, (N, K), 0.0, 0.02))
        x = synth.to_bf16_bits(synth.normal(710 + i, (M, K)))
        prob.append(dict(fmt=fmt, M=M, N=N, K=K, Wn=W, xn=x, W=to_dev(W), x=to_dev(x),
                         ws=qg.alloc_workspace(M, K, DEV),
                         y=torch.empty((M, N), dtype=torch.float32, device=DEV)))
    lm = prob[-1]
    lm_ws = qg.alloc_workspace(1, lm["K"], DEV)
    lm_y = torch.empty(lm["N"], dtype=torch.float32, device=DEV)

    def run(s):
        for p in prob:
            qg.qgemm_quantize_workspace(p["x"], p["M"], p["K"], p["ws"], s)
            qg.qgemm_gemm_quantized(p["W"], p["fmt"], p["ws"], p["M"], p["N"], p["K"], p["y"], s)
        qg.qgemm_lm_head(lm["W"], lm["fmt"], lm["x"][-1], lm["N"], lm["K"], lm_y, lm_ws, s)

    # eager reference (also warms every code path up before capture)
    with torch.cuda.stream(stream):
        run(stream)
    stream.synchronize()
    eager = [p["y"].clone() for p in prob] + [lm_y.clone()]
    for p, ye in zip(prob, eager):
        ref = oracle.gemm(p["fmt"], p["Wn"], p["xn"], p["N"])
        tol = bound(p["xn"], np.arange(p["M"]), max_abs_w(p["fmt"], p["Wn"], p["N"], p["K"]))
        check(ye.cpu().numpy(), ref, tol, f"eager fmt={p['fmt']} M={p['M']} N={p['N']} K={p['K']}")
    ref = oracle.gemm(lm["fmt"], lm["Wn"], lm["xn"], lm["N"], rows=[lm["M"] - 1])
    tol = bound(lm["xn"], [lm["M"] - 1], max_abs_w(lm["fmt"], lm["Wn"], lm["N"], lm["K"]))
    check(eager[-1].cpu().numpy()[None], ref, tol, "eager LM head")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run(stream)
    other = torch.randn(1000, 1000, device=DEV)
    for rep in range(4):
        for p in prob:
            p["y"].fill_(float("nan"))
        lm_y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        # unrelated eager work between replays, library calls included
        other = other @ other.T / 1000.0
        p0 = prob[0]
        y_side = torch.empty_like(p0["y"])
        ws_side = qg.alloc_workspace(p0["M"], p0["K"], DEV)
        qg.qgemm_prefill(p0["W"], p0["fmt"], p0["x"], p0["M"], p0["N"], p0["K"], y_side, ws_side)
        torch.cuda.synchronize()
        assert torch.equal(y_side, eager[0]), f"eager call after replay {rep}"
        for i, p in enumerate(prob):
            assert torch.equal(p["y"], eager[i]), \
                f"replay {rep}: fmt={p['fmt']} M={p['M']} N={p['N']} K={p['K']} differs from eager"
        assert torch.equal(lm_y, eager[-1]), f"replay {rep}: LM head differs from eager"


def test_graph_ffn_block_replays_match_eager():
    """One FFN block under capture: RMSNorm -> quantiser, the gate+up GEMM with
    the SwiGLU epilogue (bf16 h), the quantiser of h and the down GEMM; plus
    the fused Q5_K gate+up, the unfused SwiGLU path (Q6_K gate+up: GEMM into the
    workspace, then the SwiGLU kernel) and a Q8_0 GEMM.  Every replay equals the eager result bit
    for bit; the eager h is checked against the oracle's SwiGLU of the oracle's
    normalised rows."""
    stream = torch.cuda.Stream()
    M, F, K = 512, 3584, 1024
    xn_ = synth.to_bf16_bits(synth.student_t4(740, (M, K)))
    gn_ = synth.normal(741, (K,), 1.0, 0.25).astype(np.float32)
    Wgu_ = synth.pack(qg.QG_Q4_K, synth.normal(742, (2 * F, K), 0.0, 0.02))
    Wd_ = synth.pack(qg.QG_Q6_K, synth.normal(743, (K, F), 0.0, 0.02))
    W5_ = synth.pack(qg.QG_Q5_K, synth.normal(744, (2 * F, K), 0.0, 0.02))
    W6_ = synth.pack(qg.QG_Q6_K, synth.normal(746, (2 * F, K), 0.0, 0.02))
    W8_ = synth.pack(qg.QG_Q8_0, synth.normal(745, (700, K), 0.0, 0.02))
    x, gn, Wgu, Wd, W5, W6, W8 = (to_dev(a) for a in (xn_, gn_, Wgu_, Wd_, W5_, W6_, W8_))
    ws = torch.empty(max(qg.qgemm_swiglu_workspace_bytes(qg.QG_Q6_K, M, F, K),
                         qg.qgemm_swiglu_workspace_bytes(qg.QG_Q4_K, M, F, K)), dtype=torch.uint8, device=DEV)
    wsd = qg.alloc_workspace(M, F, DEV)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    h5 = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    h6 = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    yd = torch.empty((M, K), dtype=torch.float32, device=DEV)
    y8 = torch.empty((M, 700), dtype=torch.float32, device=DEV)
    assert qg.qgemm_kernel_name_swiglu(qg.QG_Q4_K, M, F, K).startswith("gemm_q4k_swiglu_kernel<")
    assert qg.qgemm_kernel_name_swiglu(qg.QG_Q5_K, M, F, K).startswith("gemm_q5k_swiglu_kernel<")
    assert "swiglu" not in qg.qgemm_kernel_name_swiglu(qg.QG_Q6_K, M, F, K)

    def run(s):
        qg.qgemm_rmsnorm_quantize_workspace(x, gn, 1e-6, M, K, ws, s)
        qg.qgemm_gemm_quantized_swiglu(Wgu, qg.QG_Q4_K, ws, M, F, K, h, s)
        qg.qgemm_gemm_quantized_swiglu(W5, qg.QG_Q5_K, ws, M, F, K, h5, s)
        qg.qgemm_gemm_quantized_swiglu(W6, qg.QG_Q6_K, ws, M, F, K, h6, s)
        qg.qgemm_gemm_quantized(W8, qg.QG_Q8_0, ws, M, 700, K, y8, s)
        qg.qgemm_prefill(Wd, qg.QG_Q6_K, h, M, K, F, yd, wsd, s)

    with torch.cuda.stream(stream):
        run(stream)
    stream.synchronize()
    eager = [t.clone() for t in (h, h5, h6, y8, yd)]
    # the eager h against the oracle on rows whose norm scale every summation order fixes
    r, lo, hi = oracle.rms_scale(xn_, 1e-6)
    xq = oracle.rmsnorm(xn_, gn_, r)
    rows = np.array([i for i in (0, 7, 150, 300, M - 1) if lo[i] == hi[i]])
    cols = np.array([0, 13, 777, F - 1])
    href, gref, uref = oracle.gemm_swiglu(qg.QG_Q4_K, Wgu_, xq, F, rows=rows, cols=cols)
    got = (eager[0].cpu().view(torch.int16).numpy().view(np.uint16)[np.ix_(rows, cols)].astype(np.uint32) << 16)
    got = got.view(np.float32).astype(np.float64)
    tau = bound(xq, rows, max_abs_w(qg.QG_Q4_K, Wgu_, 2 * F, K))
    pre = 1.1 * tau * (np.abs(uref) + tau) + np.abs(oracle.swiglu(gref, np.ones_like(gref))) * tau
    assert np.all(np.abs(got - href) <= pre + (2.0 ** -8 + 2.0 ** -16) * (np.abs(href) + pre) + 1e-30)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run(stream)
    for rep in range(4):
        for t in (h, h5, h6):
            t.zero_()
        y8.fill_(float("nan"))
        yd.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        # unrelated eager library work between replays
        qg.qgemm_swiglu(torch.ones((4, 16), device=DEV), 4, 8, torch.empty((4, 8), dtype=torch.bfloat16, device=DEV))
        torch.cuda.synchronize()
        for name, t, e in zip(("h", "h5", "h6", "y8", "yd"), (h, h5, h6, y8, yd), eager):
            assert torch.equal(t, e), f"replay {rep}: {name} differs from eager"
