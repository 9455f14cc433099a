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
