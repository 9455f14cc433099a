"""The C-ABI library (CPU only): it loads, exports every entry point that
include/qgemm.h declares, sizes workspaces, and rejects bad arguments with the
documented codes before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import __graft_entry__

__graft_entry__.ensure_built()
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "qgemm.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemm_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_symbols() == sorted(qg.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qg.library_path())
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_error_strings():
    for code in range(0, -9, -1):
        s = qg.qgemm_strerror(code)
        assert s and s != "unknown error code", code
    assert qg.qgemm_strerror(-99) == "unknown error code"


def test_workspace_bytes():
    ws = qg.qgemm_workspace_bytes
    assert ws(0, 256) == 0 and ws(1, 255) == 0 and ws(1, 300) == 0 and ws(-1, 256) == 0
    # rows padded to 256: int8 codes, three fp32 values and three bf16 pieces per
    # 32-value block
    per_row = lambda K: K + (K // 32) * (3 * 4 + 3 * 2)
    assert ws(1, 256) == 256 * per_row(256)
    assert ws(512, 4096) == 512 * per_row(4096)
    assert ws(513, 4096) == 768 * per_row(4096)
    assert ws(1, 1 << 40) == 0          # overflow guard


# fake but well-aligned device addresses: every call below must fail validation
# before any HIP call, so nothing is dereferenced
A = 1 << 20


def _prefill(**kw):
    lib = qg.load()
    a = dict(w=A, fmt=0, x=A, xdt=1, M=4, N=8, K=256, y=A, ws=A,
             wsb=qg.qgemm_workspace_bytes(4, 256), stream=None, path=0)
    a.update(kw)
    return lib.qgemm_prefill_ex(a["w"], a["fmt"], a["x"], a["xdt"], a["M"], a["N"], a["K"],
                                a["y"], a["ws"], a["wsb"], a["stream"], a["path"])


@pytest.mark.parametrize("kw,code", [
    (dict(w=None), -1), (dict(x=None), -1), (dict(y=None), -1),
    (dict(M=0), -1), (dict(N=0), -1), (dict(K=0), -1), (dict(K=300), -1), (dict(K=128), -1),
    (dict(M=-5), -1), (dict(N=1 << 40), -1),
    (dict(fmt=4), -2), (dict(fmt=-1), -2),
    (dict(xdt=2), -3),
    (dict(path=3), -1), (dict(path=2, M=9), -1),
    (dict(ws=None), -4), (dict(ws=A + 128), -4), (dict(wsb=100), -4),
    (dict(w=A + 8), -5), (dict(x=A + 4), -5), (dict(y=A + 4), -5),
])
def test_prefill_rejects(kw, code):
    assert _prefill(**kw) == code


def test_other_entry_points_reject():
    lib = qg.load()
    assert lib.qgemm_lm_head(None, 0, A, 1, 8, 256, A, A, 1 << 20, None) == -1
    assert lib.qgemm_lm_head(A, 7, A, 1, 8, 256, A, A, 1 << 20, None) == -2
    assert lib.qgemm_quantize_act(A, 1, 4, 48, A, A, A, None) == -1      # K % 32 != 0
    assert lib.qgemm_quantize_act(A, 5, 4, 64, A, A, A, None) == -3
    assert lib.qgemm_quantize_act(A + 2, 1, 4, 64, A, A, A, None) == -5
    assert lib.qgemm_dequant(A, 1, 8, 100, A, None) == -1
    assert lib.qgemm_dequant(A, 9, 8, 256, A, None) == -2
    assert lib.qgemm_block_partials(A, 0, None, 4, 8, 256, A, None) == -1
    assert lib.qgemm_block_partials(A, 0, A + 1, 4, 8, 256, A, None) == -5


def test_binding_refuses_host_tensors():
    import torch
    W = torch.zeros(144 * 8, dtype=torch.uint8)
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qg.prefill(W, qg.QG_Q4_K, x, 8, workspace=torch.zeros(16, dtype=torch.uint8))


def test_kernel_name_dispatch_rule():
    """Host dispatch (no GPU): which kernel each path and shape selects."""
    kn = qg.qgemm_kernel_name
    Q4, Q6, AUTO, TILED, SKINNY = qg.QG_Q4_K, qg.QG_Q6_K, qg.QG_PATH_AUTO, qg.QG_PATH_TILED, qg.QG_PATH_SKINNY
    # skinny below the measured crossover: Q6_K and Q8_0 up to 8 rows; Q4_K and
    # Q5_K up to a row count set by the shape (8 for N <= 1024; for K <= 1024, 4
    # for N <= 4096 and 2 above; otherwise 6 for N <= 12288 and 4 above)
    assert kn(Q4, 6, 4096, 4096, AUTO).startswith("skinny_kernel<0, 6,")
    assert kn(Q4, 7, 4096, 4096, AUTO).startswith("gemm_q4k_small_kernel<")
    assert kn(Q4, 8, 1024, 3584, AUTO).startswith("skinny_kernel<0, 8,")
    assert kn(Q4, 4, 4096, 1024, AUTO).startswith("skinny_kernel<0, 4,")
    assert kn(Q4, 5, 4096, 1024, AUTO).startswith("gemm_q4k_small_kernel<")
    assert kn(qg.QG_Q5_K, 2, 7168, 1024, AUTO).startswith("skinny_kernel<2, 2,")
    assert kn(qg.QG_Q5_K, 3, 7168, 1024, AUTO).startswith("gemm_q5k_small_kernel<")
    assert kn(Q4, 6, 2560, 9728, AUTO).startswith("skinny_kernel<0, 6,")
    assert kn(Q4, 7, 2560, 9728, AUTO).startswith("gemm_q4k_small_kernel<")
    assert kn(Q4, 4, 24576, 4096, AUTO).startswith("skinny_kernel<0, 4,")
    assert kn(Q4, 5, 24576, 4096, AUTO).startswith("gemm_q4k_small_kernel<")
    assert kn(qg.QG_Q8_0, 8, 4096, 4096, AUTO).startswith("skinny_kernel<3, 8,")
    assert kn(Q6, 8, 152064, 4096, AUTO).startswith("skinny_kernel<1, 8,")
    assert kn(Q6, 9, 152064, 4096, AUTO).startswith("gemm_q6k_")
    assert kn(Q4, 8, 4096, 4096, SKINNY).startswith("skinny_kernel<0, 8,")
    assert kn(Q4, 1, 4096, 4096, TILED).startswith("gemm_q4k_")
    # skinny work split: rows per step R = 16 / (K/256) when that divides, else 1;
    # activations in registers (one or two rows of K <= 4096, short rows, many rows per
    # wavefront), else in LDS whole, else one 4096-value slice of K at a time
    assert kn(Q6, 1, 152064, 4096, AUTO) == "skinny_kernel<1, 1, 1, 0, 2, 256>"
    assert kn(Q4, 2, 100, 1024, AUTO) == "skinny_kernel<0, 2, 4, 0, 0, 256>"
    assert kn(Q4, 1, 100, 2560, AUTO) == "skinny_kernel<0, 1, 1, 0, 0, 256>"
    assert kn(Q6, 8, 100, 4352, AUTO) == "skinny_kernel<1, 8, 1, 1, 0, 256>"
    assert kn(Q4, 8, 100, 12288, SKINNY) == "skinny_kernel<0, 8, 1, 2, 0, 256>"
    # Q6_K coalesced loads (last parameter: 2 straight into LDS for M <= 2,
    # 1 through registers above, 0 field loads) need aligned steps (several
    # rows per step, or rows of a multiple of 8 super-blocks), a matrix of
    # whole 16-byte chunks and the activations in registers (K <= 4096)
    assert kn(Q6, 1, 4096, 12288, AUTO) == "skinny_kernel<1, 1, 1, 1, 0, 256>"
    assert kn(Q6, 1, 77, 1024, AUTO) == "skinny_kernel<1, 1, 4, 0, 0, 256>"    # 77*4 % 8 != 0
    assert kn(Q6, 2, 78, 1024, AUTO) == "skinny_kernel<1, 2, 4, 0, 2, 256>"
    assert kn(Q6, 1, 80, 2560, AUTO) == "skinny_kernel<1, 1, 1, 0, 0, 256>"    # 10 super-blocks a row
    assert kn(Q6, 3, 81, 2048, AUTO) == "skinny_kernel<1, 3, 2, 0, 1, 256>"
    assert kn(Q6, 1, 80, 4096, AUTO) == "skinny_kernel<1, 1, 1, 0, 0, 256>"  # field loads at N <= 16384
    assert kn(Q6, 8, 152064, 4096, AUTO) == "skinny_kernel<1, 8, 1, 0, 1, 512>"  # from M = 5: 512 threads
    assert kn(Q6, 5, 152064, 4096, AUTO) == "skinny_kernel<1, 5, 1, 0, 1, 512>"
    assert kn(Q6, 4, 152064, 4096, AUTO) == "skinny_kernel<1, 4, 1, 0, 1, 256>"
    # from three rows of K > 2048 the activations go to LDS unless each
    # wavefront takes many rows (N > 16384)
    assert kn(Q6, 8, 2560, 4096, AUTO) == "skinny_kernel<1, 8, 1, 1, 0, 256>"
    assert kn(Q4, 4, 9728, 2560, AUTO) == "skinny_kernel<0, 4, 1, 1, 0, 512>"
    assert kn(Q4, 4, 24576, 4096, AUTO) == "skinny_kernel<0, 4, 1, 0, 0, 256>"
    # launch plans (last parameter: threads per workgroup) for Q4_K and Q6_K rows
    # of one step or more: 1024 for whole rows of K > 4096 in LDS over at least
    # 2048 weight rows, 512 for rows of K <= 4096 in LDS over at least 8192
    # weight rows and for slices over a multiple of 4096 weight rows from M = 6
    assert kn(Q6, 4, 4096, 12288, AUTO) == "skinny_kernel<1, 4, 1, 1, 0, 1024>"
    assert kn(Q6, 8, 4096, 12288, AUTO) == "skinny_kernel<1, 8, 1, 2, 0, 512>"
    assert kn(Q6, 5, 4096, 12288, AUTO) == "skinny_kernel<1, 5, 1, 2, 0, 256>"
    assert kn(Q4, 5, 2560, 9728, AUTO) == "skinny_kernel<0, 5, 1, 1, 0, 1024>"
    assert kn(Q6, 2, 1000, 12288, AUTO) == "skinny_kernel<1, 2, 1, 1, 0, 256>"
    assert kn(Q4, 6, 2560, 9728, AUTO) == "skinny_kernel<0, 6, 1, 2, 0, 256>"
    assert kn(qg.QG_Q5_K, 4, 2560, 9728, AUTO) == "skinny_kernel<2, 4, 1, 1, 0, 256>"
    assert kn(qg.QG_Q5_K, 4, 9728, 2560, AUTO) == "skinny_kernel<2, 4, 1, 1, 0, 512>"
    assert kn(qg.QG_Q8_0, 8, 9728, 2560, AUTO) == "skinny_kernel<3, 8, 1, 1, 0, 512>"
    assert kn(Q6, 5, 151936, 2560, AUTO) == "skinny_kernel<1, 5, 1, 0, 0, 256>"  # unaligned: field loads
    assert kn(Q6, 5, 16400, 4096, AUTO) == "skinny_kernel<1, 5, 1, 0, 1, 512>"
    # decode-sized batches on the small-grid kernel: four epilogue rows per
    # lane, about 1024 waves
    assert kn(Q4, 8, 24576, 4096, AUTO) == "gemm_q4k_small_kernel<2, 4>"
    assert kn(Q4, 8, 9728, 2560, AUTO) == "gemm_q4k_small_kernel<4, 4>"
    assert kn(Q4, 9, 9728, 2560, AUTO) == "gemm_q4k_small_kernel<8, 16>"
    # tiled tile choice by grid size
    assert kn(Q4, 8192, 24576, 4096, AUTO) == "gemm_q4k_lds_kernel<2, 2, 2, 4, false, 2, 2, 1, false>"
    # one round of 128x256 blocks plus 64x256 blocks over the other columns
    # (512 rows: 256 + 256 blocks), where 128x256 blocks alone would leave a
    # second round half empty
    assert kn(Q4, 512, 24576, 4096, AUTO) == "gemm_q4k_mix_kernel"
    assert kn(Q4, 500, 20500, 768, AUTO) == "gemm_q4k_mix_kernel"
    assert kn(Q4, 256, 45000, 512, AUTO) == "gemm_q4k_mix_kernel"
    assert kn(Q4, 300, 20500, 768, AUTO) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, false>"  # 3 row tiles
    assert kn(Q4, 512, 18000, 4096, AUTO) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, false>"  # short 2nd round
    assert qg.qgemm_kernel_name_a256(0, 512, 24576, 4096) != "gemm_q4k_mix_kernel"
    # long prompts: 128x256 blocks unless their last round is much emptier than 64x128's
    big, mid = ("gemm_q4k_lds_kernel<2, 2, 2, 4, false, 2, 2, 1, false>",
                "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, false>")
    assert kn(Q4, 2048, 24576, 4096, AUTO) == big and kn(Q4, 8192, 24576, 4096, AUTO) == big
    assert kn(Q4, 4096, 9728, 2560, AUTO) == big
    # 320 large blocks on 256 CUs: one round of them, the other columns in 128 64x256 blocks
    assert kn(Q4, 4096, 2560, 9728, AUTO) == "gemm_q4k_mix_kernel"
    assert kn(Q4, 3000, 2560, 9728, AUTO) == mid      # 24 row tiles: no whole round of large blocks
    assert kn(Q4, 64, 1024, 1024, AUTO).startswith("gemm_q4k_small_kernel<")
    # few output blocks: K split inside the workgroup
    assert kn(Q4, 512, 2560, 9728, AUTO) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 2, false>"
    assert kn(Q4, 512, 1024, 3584, AUTO) == "gemm_q4k_lds_kernel<1, 1, 1, 2, false, 2, 2, 4, false>"
    assert kn(Q4, 330, 2700, 1280, AUTO) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 2, false>"
    assert kn(Q4, 170, 2800, 2816, AUTO) == "gemm_q4k_lds_kernel<1, 1, 1, 2, false, 2, 2, 4, false>"
    assert kn(Q4, 512, 1024, 1792, AUTO).startswith("gemm_q4k_small_kernel<")   # too few super-blocks
    # Q6_K: 128x128 blocks when their grid fills whole rounds (or many), else
    # the half-stage kernel at 64x64, or 64x64 with a split K range
    q6big = "gemm_q6k_lds_kernel<2, 1, 2, 4, 2, 2, 1>"
    assert kn(Q6, 8192, 4096, 12288, AUTO) == q6big and kn(Q6, 2048, 4096, 12288, AUTO) == q6big
    assert kn(Q6, 1024, 4096, 12288, AUTO) == q6big                     # 256 blocks: one round
    assert kn(Q6, 512, 152064, 4096, AUTO) == q6big                      # 4752 blocks
    half = "gemm_q6k_half_kernel<1, 1, 2, 2, 2, 4, 1>"
    assert kn(Q6, 4096, 2560, 4096, AUTO) == half                        # 640 blocks: 2.5 rounds
    assert kn(Q6, 1536, 4096, 12288, AUTO) == half
    assert kn(Q6, 512, 4096, 12288, AUTO) == half and kn(Q6, 512, 2560, 4096, AUTO) == half
    assert kn(Q6, 77, 300, 1024, AUTO) == "gemm_q6k_half_kernel<1, 1, 2, 2, 2, 4, 2>"
    assert kn(Q6, 70, 300, 256, AUTO) == half
    # arguments the entry points would reject
    assert kn(4, 8, 8, 256, AUTO) is None
    assert kn(Q4, 8, 8, 300, AUTO) is None
    assert kn(Q4, 9, 8, 256, SKINNY) is None
    assert kn(Q4, 0, 8, 256, AUTO) is None


def test_a256_host_side():
    """Per-256 entry points: argument checks and kernel choice (no GPU call)."""
    lib = qg.load()
    wsb = qg.qgemm_workspace_bytes(4, 256)
    call = lambda **k: lib.qgemm_prefill_a256(
        k.get("w", A), k.get("fmt", 0), k.get("x", A), k.get("xdt", 1), k.get("M", 4),
        k.get("N", 8), k.get("K", 256), k.get("y", A), k.get("ws", A), k.get("wsb", wsb), None)
    assert call(w=None) == -1 and call(M=0) == -1 and call(K=300) == -1
    assert call(fmt=1) == -2 and call(xdt=3) == -3
    assert call(ws=None) == -4 and call(wsb=wsb - 1) == -4
    assert call(x=A + 2) == -5 and call(y=A + 4) == -5
    assert lib.qgemm_quantize_act_a256(A, 1, 4, 288, A, A, A, None) == -1   # K % 256 != 0
    assert lib.qgemm_quantize_act_a256(A, 1, 4, 512, A, A + 2, A, None) == -5
    kn = qg.qgemm_kernel_name_a256
    assert kn(1, 512, 4096, 1024) is None
    assert kn(0, 512, 24576, 4096) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, true>"
    assert kn(0, 8192, 24576, 4096) == "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, true>"
    assert kn(0, 64, 1024, 1024).startswith("gemm_q4k_small_kernel<")
    assert kn(0, 3, 300, 1024).startswith("skinny_kernel<0, 3,")


def test_deq_f16_branch_host_side():
    """The dequantise-to-fp16 branch: workspace sizing, argument checks and kernel
    choice (no GPU call)."""
    lib = qg.load()
    ws = qg.qgemm_deq_f16_workspace_bytes
    assert ws(0, 256) == 0 and ws(4, 300) == 0 and ws(1, 1 << 40) == 0
    assert ws(1, 256) == 512 and ws(3, 256) == 1536 and ws(5, 256) == 2560
    assert ws(512, 4096) == 512 * 4096 * 2
    wsb = ws(4, 256)
    call = lambda **k: lib.qgemm_prefill_deq_f16(
        k.get("w", A), k.get("fmt", 0), k.get("x", A), k.get("xdt", 1), k.get("M", 4),
        k.get("N", 8), k.get("K", 256), k.get("y", A), k.get("ws", A), k.get("wsb", wsb), None)
    assert call(w=None) == -1 and call(M=0) == -1 and call(K=300) == -1
    assert call(fmt=2) == -2 and call(fmt=5) == -2
    assert call(xdt=3) == -3
    assert call(ws=None) == -4 and call(wsb=wsb - 1) == -4 and call(ws=A + 64) == -4
    assert call(x=A + 2) == -5 and call(y=A + 4) == -5 and call(w=A + 8) == -5
    assert lib.qgemm_to_f16(A, 1, 4, 12, A, None) == -1     # K % 8 != 0
    assert lib.qgemm_to_f16(A, 4, 4, 16, A, None) == -3
    assert lib.qgemm_to_f16(A, 1, 4, 16, A + 2, None) == -5
    assert lib.qgemm_dequant_f16(A, 0, 8, 100, A, None) == -1
    assert lib.qgemm_dequant_f16(A, 2, 8, 256, A, None) == -2
    assert lib.qgemm_dequant_f16(A, 0, 8, 256, A + 2, None) == -5
    kn = qg.qgemm_deq_f16_kernel_name
    assert kn(2, 512, 4096, 1024) is None and kn(0, 512, 4096, 1000) is None
    assert kn(0, 512, 24576, 4096) == "gemm_deq_f16_kernel<0, 4, 1, 2, 8, 2, 4, 1>"
    assert kn(0, 2048, 24576, 4096) == "gemm_deq_f16_kernel<0, 4, 1, 2, 8, 2, 4, 1>"
    assert kn(0, 4096, 2560, 9728) == "gemm_deq_f16_kernel<0, 4, 1, 2, 8, 2, 4, 1>"
    assert kn(0, 4096, 9728, 2560) == "gemm_deq_f16_kernel<0, 4, 1, 2, 4, 2, 4, 1>"
    assert kn(0, 700, 11000, 512) == "gemm_deq_f16_kernel<0, 4, 1, 2, 4, 2, 4, 1>"
    assert kn(0, 512, 7168, 1024) == "gemm_deq_f16_kernel<0, 4, 1, 1, 4, 2, 4, 1>"
    # smaller grids split K inside the workgroup
    assert kn(0, 512, 4096, 1024) == "gemm_deq_f16_kernel<0, 2, 1, 1, 4, 2, 4, 2>"
    assert kn(0, 512, 2560, 9728) == "gemm_deq_f16_kernel<0, 4, 1, 1, 2, 2, 2, 4>"
    assert kn(0, 512, 1024, 3584) == "gemm_deq_f16_kernel<0, 1, 1, 1, 2, 2, 4, 4>"
    assert kn(0, 1, 77, 256) == "gemm_deq_f16_kernel<0, 1, 1, 1, 2, 2, 4, 4>"
    # Q6_K: the same large blocks; small grids take 128x64 blocks with three K-groups
    assert kn(1, 512, 4096, 12288) == "gemm_deq_f16_kernel<1, 4, 1, 1, 2, 2, 2, 3>"
    assert kn(1, 512, 2560, 4096) == "gemm_deq_f16_kernel<1, 4, 1, 1, 2, 2, 2, 3>"
    assert kn(1, 64, 1024, 1024) == "gemm_deq_f16_kernel<1, 1, 1, 1, 2, 2, 4, 4>"
    assert kn(1, 8192, 4096, 12288) == "gemm_deq_f16_kernel<1, 4, 1, 2, 8, 2, 4, 1>"


def test_fusion_host_side():
    """RMSNorm -> quantiser and the SwiGLU entry points: workspace sizing,
    argument checks and kernel choice (no GPU call)."""
    lib = qg.load()
    wsz = qg.qgemm_swiglu_workspace_bytes
    base = qg.qgemm_workspace_bytes
    assert wsz(0, 512, 12288, 4096) == base(512, 4096)            # fused: no fp32 scratch
    assert wsz(0, 512, 3584, 1024) == base(512, 1024)
    assert wsz(1, 512, 1536, 4096) == base(512, 4096) + 512 * 3072 * 4   # Q6_K: GEMM + SwiGLU kernel
    assert wsz(0, 3, 1000, 256) == base(3, 256) + (3 * 2000 * 4 + 255) // 256 * 256  # skinny
    assert wsz(4, 4, 8, 256) == 0 and wsz(0, 0, 8, 256) == 0 and wsz(0, 4, 0, 256) == 0
    assert wsz(0, 4, 8, 300) == 0
    kn = qg.qgemm_kernel_name_swiglu
    assert kn(0, 512, 3584, 1024) == "gemm_q4k_swiglu_kernel<1, 1, 2, 4, 2, 4, 1>"
    assert kn(0, 512, 12288, 4096) == "gemm_q4k_swiglu_mix_kernel"   # 128x256 then 64x256 blocks
    assert kn(0, 512, 9000, 4096) == "gemm_q4k_swiglu_kernel<1, 1, 2, 4, 2, 4, 1>"   # short second round
    assert kn(0, 8192, 12288, 4096) == "gemm_q4k_swiglu_kernel<2, 2, 2, 4, 2, 2, 1>"
    assert kn(0, 64, 512, 1024).startswith("gemm_q4k_small_kernel<")
    assert kn(0, 3, 1000, 256).startswith("skinny_kernel<0, 3,")
    assert kn(1, 512, 1536, 4096).startswith("gemm_q6k_")
    assert kn(4, 512, 8, 256) is None and kn(0, 512, 8, 300) is None
    wsb = wsz(0, 4, 8, 256)
    call = lambda **k: lib.qgemm_prefill_swiglu(
        k.get("w", A), k.get("fmt", 0), k.get("x", A), k.get("xdt", 1), k.get("M", 4),
        k.get("F", 8), k.get("K", 256), k.get("h", A), k.get("ws", A), k.get("wsb", wsb), None)
    assert call(w=None) == -1 and call(M=0) == -1 and call(F=0) == -1 and call(K=300) == -1
    assert call(h=None) == -1 and call(fmt=4) == -2 and call(xdt=3) == -3
    assert call(ws=None) == -4 and call(wsb=wsb - 1) == -4
    assert call(x=A + 2) == -5 and call(h=A + 2) == -5
    assert lib.qgemm_gemm_quantized_swiglu(A, 0, A, wsb, 4, 8, 256, A + 8, None) == -5
    assert lib.qgemm_swiglu(A, 4, 0, A, None) == -1 and lib.qgemm_swiglu(A + 4, 4, 8, A, None) == -5
    rbytes = base(4, 512)
    rms = lambda **k: lib.qgemm_rmsnorm_quantize_workspace(
        k.get("x", A), k.get("xdt", 1), k.get("g", A), k.get("eps", 1e-6), k.get("M", 4), k.get("K", 512),
        k.get("ws", A), k.get("wsb", rbytes), None)
    assert rms(x=None) == -1 and rms(g=None) == -1 and rms(M=0) == -1 and rms(K=300) == -1
    assert rms(K=65536) == -1 and rms(eps=-1e-6) == -1 and rms(eps=float("nan")) == -1
    assert rms(eps=float("inf")) == -1 and rms(M=1 << 31) == -1
    assert rms(xdt=3) == -3 and rms(g=A + 4) == -5 and rms(x=A + 2) == -5
    assert rms(ws=None) == -4 and rms(wsb=rbytes - 1) == -4
    assert lib.qgemm_rmsnorm_quantize_act(A, 1, A, 1e-6, 4, 512, A, A + 2, A, None) == -5


def test_q5k_host_side():
    """Q5_K: kernel choice, its workspace-free SwiGLU fallback, and the entry
    points that do not take it (no GPU call)."""
    kn = qg.qgemm_kernel_name
    assert kn(2, 512, 4096, 1024) == "gemm_q5k_lds_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert kn(2, 8192, 24576, 4096) == "gemm_q5k_lds_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert kn(2, 512, 1024, 3584) == "gemm_q5k_lds_kernel<1, 1, 1, 2, 2, 2, 3>"
    assert kn(2, 64, 1024, 1024).startswith("gemm_q5k_small_kernel<")
    assert kn(2, 1, 24576, 4096) == "skinny_kernel<2, 1, 1, 0, 0, 256>"
    assert kn(2, 4, 4096, 1024).startswith("skinny_kernel<2, 4,")
    assert kn(2, 5, 4096, 1024).startswith("gemm_q5k_small_kernel<")
    assert kn(2, 6, 2560, 9728).startswith("skinny_kernel<2, 6,")
    assert kn(2, 7, 2560, 9728).startswith("gemm_q5k_small_kernel<")
    assert kn(2, 8, 4096, 1024, qg.QG_PATH_SKINNY).startswith("skinny_kernel<2, 8,")
    assert qg.qgemm_kernel_name_swiglu(2, 512, 3584, 1024) == "gemm_q5k_swiglu_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert qg.qgemm_swiglu_workspace_bytes(2, 512, 3584, 1024) == qg.qgemm_workspace_bytes(512, 1024)
    assert qg.qgemm_kernel_name_swiglu(2, 64, 512, 1024).startswith("gemm_q5k_small_kernel<")  # not fused
    assert qg.qgemm_swiglu_workspace_bytes(2, 64, 512, 1024) == \
        qg.qgemm_workspace_bytes(64, 1024) + 64 * 1024 * 4
    lib = qg.load()
    ws = qg.qgemm_workspace_bytes(4, 256)
    assert lib.qgemm_prefill_a256(A, 2, A, 1, 4, 8, 256, A, A, ws, None) == -2
    assert lib.qgemm_prefill_deq_f16(A, 2, A, 1, 4, 8, 256, A, A, 1 << 20, None) == -2
    assert lib.qgemm_dequant_f16(A, 2, 8, 256, A, None) == -2
    assert qg.qgemm_kernel_name_a256(2, 512, 4096, 1024) is None


def test_q80_host_side():
    """Q8_0: kernel choice and the entry points that do not take it (no GPU call)."""
    kn = qg.qgemm_kernel_name
    assert kn(3, 512, 4096, 1024) == "gemm_q80_lds_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert kn(3, 8192, 24576, 4096) == "gemm_q80_lds_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert kn(3, 512, 1024, 3584) == "gemm_q80_lds_kernel<1, 1, 1, 2, 2, 2, 3>"
    assert kn(3, 64, 1024, 512) == "gemm_q80_lds_kernel<1, 1, 1, 2, 2, 2, 1>"
    assert kn(3, 1, 24576, 4096) == "skinny_kernel<3, 1, 1, 0, 0, 256>"
    assert kn(3, 8, 4096, 1024, qg.QG_PATH_SKINNY).startswith("skinny_kernel<3, 8,")
    assert qg.qgemm_kernel_name_swiglu(3, 512, 3584, 1024) == "gemm_q80_swiglu_kernel<1, 1, 2, 4, 2, 2, 1>"
    assert qg.qgemm_kernel_name_swiglu(3, 300, 700, 768) == "gemm_q80_swiglu_kernel<1, 1, 1, 2, 2, 2, 3>"
    assert qg.qgemm_kernel_name_swiglu(3, 8, 700, 768).startswith("skinny_kernel<3, 8,")
    lib = qg.load()
    assert lib.qgemm_prefill_a256(A, 3, A, 1, 4, 8, 256, A, A, 1 << 20, None) == -2
    assert lib.qgemm_prefill_deq_f16(A, 3, A, 1, 4, 8, 256, A, A, 1 << 20, None) == -2
    assert lib.qgemm_dequant_f16(A, 3, 8, 256, A, None) == -2


def test_sclk_probe_rejects_bad_arguments():
    lib = qg.load()
    assert lib.qgemm_sclk_probe(None, 10, None) == -1
    assert lib.qgemm_sclk_probe(A, 0, None) == -1
    assert lib.qgemm_sclk_probe(A, (1 << 24) + 1, None) == -1
    assert lib.qgemm_sclk_probe(A + 4, 10, None) == -5


def test_read_probe_rejects_bad_arguments():
    lib = qg.load()
    assert lib.qgemm_read_probe(A, -16, None) == -1
    assert lib.qgemm_read_probe(A, 24, None) == -1
    assert lib.qgemm_read_probe(None, 16, None) == -1
    assert lib.qgemm_read_probe(A + 8, 16, None) == -5


def test_plant_delay_host_side():
    """The timing falsifier's planted delay: host-side state only, bounded."""
    lib = qg.load()
    hdr = open(HEADER).read()
    assert f"#define QG_PLANT_QUANTIZE {qg.QG_PLANT_QUANTIZE}" in hdr
    assert f"#define QG_PLANT_MAX_SLEEPS {qg.QG_PLANT_MAX_SLEEPS}" in hdr
    assert lib.qgemm_test_plant_delay(0, 10) == -1
    assert lib.qgemm_test_plant_delay(2, 10) == -1
    assert lib.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, -1) == -1
    assert lib.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, qg.QG_PLANT_MAX_SLEEPS + 1) == -1
    try:
        assert lib.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, qg.QG_PLANT_MAX_SLEEPS) == 0
    finally:
        assert lib.qgemm_test_plant_delay(qg.QG_PLANT_QUANTIZE, 0) == 0


def test_library_matches_its_sources():
    """The in-tree library was built from the sources the tree holds (the binding
    refuses a stale one)."""
    from quantized_prefill_gemm_q8_amd import _build
    info = _build.build_info()
    assert info.get("source_sha256") == _build.source_sha256()
    assert not _build.is_stale()


def test_noalloc_rejects_before_any_launch():
    lib = qg.load()
    f = lib.qgemm_prefill_noalloc
    assert f(None, 0, A, 1, 1, 1, 256, A, None) == -1
    assert f(A, 0, A, 1, 1, 1, 300, A, None) == -1
    assert f(A, 0, A, 1, 0, 1, 256, A, None) == -1
    # 4096 x 4096 needs 26 MB of workspace: more than the static 16 MiB
    assert qg.qgemm_workspace_bytes(4096, 4096) > qg.QG_NOALLOC_SCRATCH_BYTES
    assert f(A, 0, A, 1, 4096, 256, 4096, A, None) == qg.QG_ENOSCRATCH


def test_skinny_plans_are_built():
    """Every skinny kernel the dispatch names is one the library builds: 512
    threads with the activations staged in LDS (any format) or in slices (Q4_K,
    Q6_K), without coalesced loads, or for Q6_K with the coalesced loads through
    registers; 1024 threads with whole rows in LDS (Q4_K, Q6_K); both only for
    rows of one step or more."""
    Ks = [256, 512, 1024, 2048, 2560, 3072, 3584, 4096, 4352, 6144, 8192, 9728, 12288]
    Ns = [77, 80, 1000, 2048, 2560, 4096, 8192, 9728, 16384, 16400, 24576, 151936, 152064]
    seen = set()
    for fmt in (qg.QG_Q4_K, qg.QG_Q6_K, qg.QG_Q5_K, qg.QG_Q8_0):
        for M in range(1, qg.QG_SKINNY_MAX_M + 1):
            for K in Ks:
                for N in Ns:
                    name = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_SKINNY)
                    f, m, r, xm, co, th = (int(v) for v in name[len("skinny_kernel<"):-1].split(","))
                    assert (f, m) == (fmt, M), name
                    assert r == (16 // (K // 256) if K // 256 in (1, 2, 4, 8) else 1), name
                    if xm == 2:
                        assert r == 1 and co == 0, name
                    if co != 0:
                        assert fmt == qg.QG_Q6_K and xm == 0, name
                    if th == 512:
                        assert r == 1, name
                        assert ((xm in (1, 2) and co == 0 and (xm == 1 or fmt in (qg.QG_Q4_K, qg.QG_Q6_K)))
                                or (xm == 0 and co == 1)), name
                    elif th == 1024:
                        assert fmt in (qg.QG_Q4_K, qg.QG_Q6_K) and r == 1 and xm == 1 and co == 0, name
                    else:
                        assert th == 256, name
                    seen.add(th)
    assert seen == {256, 512, 1024}, seen
