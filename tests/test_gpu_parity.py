"""GPU parity: libqgemm.so (through its C ABI) against the CPU oracle.

Bit-exact: activation codes, scales and block sums; decoded weights (as the
correctly rounded fp32 of the exact value); per-block int32 partials.  Within
the acceptance bound |dy| <= 1e-3 * ||x_row||_2 * max|w|: the GEMM output, on
every element at small sizes and on sampled elements at the workloads' full
sizes.  Plus the exact cases (textbook integer matmul, power-of-two scaling,
row-split and run-to-run identity) and the edge shapes.
"""
import numpy as np
import pytest
import torch

import __graft_entry__

__graft_entry__.ensure_built()
import oracle  # noqa: E402
import synth  # noqa: E402
import quantized_prefill_gemm_q8_amd as qg  # noqa: E402
from gpu_util import DEV, bound, check, max_abs_w, to_dev, x_as_f32  # noqa: E402
import pins  # noqa: E402

pytestmark = pytest.mark.gpu

FMTS = [qg.QG_Q4_K, qg.QG_Q6_K, qg.QG_Q5_K, qg.QG_Q8_0]
FMT_ID = {qg.QG_Q4_K: "q4k", qg.QG_Q6_K: "q6k", qg.QG_Q5_K: "q5k", qg.QG_Q8_0: "q80"}


def gpu_prefill(W: np.ndarray, fmt: int, x: np.ndarray, N: int, path=qg.QG_PATH_AUTO) -> np.ndarray:
    y = qg.prefill(to_dev(W), fmt, to_dev(x), N, path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------------ quantiser

def _special_rows(K):
    rows = []
    r = np.zeros(K, np.float32); rows.append(r)                                  # all zero
    r = synth.normal(501, K); r[:32] = 0; r[64:96] = -0.0; rows.append(r)       # zero blocks
    r = np.float32(2.0 ** -140) * synth.normal(502, K); rows.append(r.astype(np.float32))  # subnormal
    r = np.float32(1e-37) * synth.normal(503, K); rows.append(r.astype(np.float32))  # tiny normal
    r = np.float32(1e30) * synth.normal(504, K); rows.append(r.astype(np.float32))   # huge
    r = np.tile(np.float32([127, 0.5, 1.5, 2.5, -0.5, -2.5, 126.5, -3.5]), K // 8); rows.append(r)  # ties
    r = synth.normal(505, K); r[::32] *= 1000; rows.append(r)                    # block outliers
    r = np.full(K, 1.0, np.float32); rows.append(r)                              # all ones
    r = np.full(K, 2.0 ** -149, np.float32); r[1::2] *= -1; rows.append(r)      # min subnormal
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_act_bitexact(dtype):
    M, K = 37, 1024
    x = synth.normal(510, (M, K))
    x[::5] *= np.float32(8.0)
    x = np.concatenate([x, _special_rows(K)])
    if dtype == "bf16":
        x = synth.to_bf16_bits(x)
    M = x.shape[0]
    xq, xd, xs = oracle.quantize_act(x)
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    d = torch.empty((M, K // 32), dtype=torch.float32, device=DEV)
    S = torch.empty((M, K // 32), dtype=torch.int32, device=DEV)
    qg.qgemm_quantize_act(to_dev(x), M, K, q, d, S)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), xq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), xd.view(np.uint32))
    assert np.array_equal(S.cpu().numpy(), xs)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_quantize_act_bitexact_config_rows(cfg):
    g = synth.CONFIGS[cfg][0]
    x = synth.make_acts(g, rows=min(g.M, 64))
    M, K = x.shape
    xq, xd, xs = oracle.quantize_act(x)
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    d = torch.empty((M, K // 32), dtype=torch.float32, device=DEV)
    S = torch.empty((M, K // 32), dtype=torch.int32, device=DEV)
    qg.qgemm_quantize_act(to_dev(x), M, K, q, d, S)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), xq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), xd.view(np.uint32))
    assert np.array_equal(S.cpu().numpy(), xs)


# ------------------------------------------------------------------ decoders

@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
@pytest.mark.parametrize("kind", ["packed", "random", "random_subnormal"])
def test_dequant_bitexact(fmt, kind):
    N, K = 33, 768
    if kind == "packed":
        W = synth.pack(fmt, synth.normal(520 + fmt, (N, K), 0.0, 0.02))
    elif kind == "random":
        W = synth.random_blocks(fmt, N, K, seed=521 + fmt, emin=1, emax=30)
    else:
        W = synth.random_blocks(fmt, N, K, seed=522 + fmt, emin=0, emax=3)
    w = torch.empty((N, K), dtype=torch.float32, device=DEV)
    qg.qgemm_dequant(to_dev(W), fmt, N, K, w)
    torch.cuda.synchronize()
    ref = oracle.dequant(fmt, W, N, K).astype(np.float32)
    got = w.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"{np.sum(got != ref)} of {got.size} decoded weights differ"


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
@pytest.mark.parametrize("shape", [(37, 45, 512), (64, 64, 256), (1, 1, 256), (65, 97, 768)])
def test_block_partials_bitexact(fmt, shape):
    M, N, K = shape
    W = synth.random_blocks(fmt, N, K, seed=530 + M + fmt, emin=1, emax=20)
    rng = np.random.default_rng(531 + N)
    qx = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    qx[:, ::32] = 127
    qx[0, :] = -128
    L = 16 if fmt == qg.QG_Q6_K else 32
    out = torch.empty((M, N, K // L), dtype=torch.int32, device=DEV)
    qg.qgemm_block_partials(to_dev(W), fmt, to_dev(qx), M, N, K, out)
    torch.cuda.synchronize()
    ref = oracle.block_partials(fmt, W, qx, N)
    got = out.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} of {got.size} partials differ"


# ------------------------------------------------------------------ GEMM: small, every element

@pytest.mark.parametrize("path", [qg.QG_PATH_AUTO, qg.QG_PATH_TILED])
@pytest.mark.parametrize("cfg_idx", [(1, 0), (2, 0), (2, 1), (2, 2)],
                         ids=lambda c: f"config{c[0]}_{synth.CONFIGS[c[0]][c[1]].name}")
def test_gemm_small_configs_every_element(cfg_idx, path):
    g = synth.CONFIGS[cfg_idx[0]][cfg_idx[1]]
    W = synth.make_weights(g)
    x = synth.make_acts(g)
    y = gpu_prefill(W, g.fmt, x, g.N, path)
    ref = oracle.gemm(g.fmt, W, x, g.N)
    tol = bound(x, np.arange(g.M), max_abs_w(g.fmt, W, g.N, g.K))
    r = check(y, ref, tol, g.name)
    print(f"{g.name}: max err/tol {r:.2e}")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
@pytest.mark.parametrize("N", [1, 31, 33, 1000])
def test_gemm_edge_shapes(fmt, N):
    K = 256 if N != 33 else 1280
    W = synth.pack(fmt, synth.normal(540 + N, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    for M in (1, 2, 3, 5, 8, 9, 63, 65, 511, 513):
        x = synth.to_bf16_bits(synth.normal(541 + M, (M, K)))
        ref = oracle.gemm(fmt, W, x, N)
        tol = bound(x, np.arange(M), wmax)
        paths = [qg.QG_PATH_TILED] + ([qg.QG_PATH_SKINNY] if M <= qg.QG_SKINNY_MAX_M else [])
        for p in paths:
            check(gpu_prefill(W, fmt, x, N, p), ref, tol, f"M={M} N={N} K={K} path={p}")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
def test_gemm_random_blocks(fmt):
    """Random legal blocks: negative scales, saturating codes, subnormal binary16."""
    M, N, K = 70, 130, 512
    W = synth.random_blocks(fmt, N, K, seed=550 + fmt, emin=0, emax=16)
    x = synth.normal(551, (M, K))
    ref = oracle.gemm(fmt, W, x, N)
    tol = bound(x, np.arange(M), max_abs_w(fmt, W, N, K))
    for p in (qg.QG_PATH_TILED,):
        check(gpu_prefill(W, fmt, x, N, p), ref, tol, f"random blocks path={p}")
    check(gpu_prefill(W, fmt, x[:7].copy(), N, qg.QG_PATH_SKINNY), ref[:7], tol[:7], "skinny")


# ------------------------------------------------------------------ exact cases

@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
@pytest.mark.parametrize("path", [qg.QG_PATH_TILED, qg.QG_PATH_SKINNY])
def test_textbook_integer_matmul_exact(fmt, path):
    M = 37 if path == qg.QG_PATH_TILED else 8
    N, K = 70, 1024
    W, wv = pins._textbook_blocks(fmt, N, K, seed=560 + fmt)
    xi = pins._integer_acts(M, K, seed=561)
    y = gpu_prefill(W, fmt, xi.astype(np.float32), N, path)
    exact = (xi @ wv.T).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), exact), np.abs(y - exact).max()


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
def test_worked_examples_all_ones(fmt):
    blk, fx = {qg.QG_Q4_K: pins.q4k_example_block, qg.QG_Q5_K: pins.q5k_example_block,
               qg.QG_Q6_K: pins.q6k_example_block, qg.QG_Q8_0: pins.q80_example_block}[fmt]()
    if fmt == qg.QG_Q8_0:                   # one 256-value row: eight copies of the 32-value block
        blk, fx = np.tile(blk, 8), dict(fx, sum_w=8 * float(fx["sum_w"]))
    x = np.ones((3, 256), np.float32)
    ref = oracle.gemm(fmt, blk, x, 1)
    for p in (qg.QG_PATH_TILED, qg.QG_PATH_SKINNY):
        y = gpu_prefill(blk, fmt, x, 1, p)
        tol = bound(x, np.arange(3), max_abs_w(fmt, blk, 1, 256))
        check(y, ref, tol, f"worked example path={p}")
        assert np.allclose(y[:, 0], float(fx["sum_w"]), rtol=1e-6)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
def test_invariants(fmt):
    M, N, K = 100, 96, 1024
    W = synth.pack(fmt, synth.normal(570 + fmt, (N, K), 0.0, 0.02))
    x = synth.normal(571, (M, K))
    y = gpu_prefill(W, fmt, x, N, qg.QG_PATH_TILED)
    # run-to-run identity (no atomics, fixed order)
    assert np.array_equal(y, gpu_prefill(W, fmt, x, N, qg.QG_PATH_TILED))
    # a row depends only on its own input row: any split of M gives identical rows
    ys = np.concatenate([gpu_prefill(W, fmt, x[a:b].copy(), N, qg.QG_PATH_TILED)
                         for a, b in ((0, 33), (33, 34), (34, 100))])
    assert np.array_equal(ys, y)
    # power-of-two scaling of x scales y exactly
    for k in (-7, 3):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(gpu_prefill(W, fmt, xs, N, qg.QG_PATH_TILED), y * np.float32(2.0 ** k))
    # zero rows give zero outputs
    xz = x.copy(); xz[5] = 0
    assert np.all(gpu_prefill(W, fmt, xz, N, qg.QG_PATH_TILED)[5] == 0)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
def test_lm_head_matches_prefill_last_row(fmt):
    M, N, K = 40, 500, 1024
    W = synth.pack(fmt, synth.normal(580 + fmt, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(581, (M, K)))
    y = gpu_prefill(W, fmt, x, N)
    xd = to_dev(x)
    ws = qg.alloc_workspace(1, K, DEV)
    yl = torch.empty(N, dtype=torch.float32, device=DEV)
    qg.qgemm_lm_head(to_dev(W), fmt, xd[M - 1], N, K, yl, ws)
    torch.cuda.synchronize()
    ref = oracle.gemm(fmt, W, x, N, rows=[M - 1])
    tol = bound(x, [M - 1], max_abs_w(fmt, W, N, K))
    check(yl.cpu().numpy()[None], ref, tol, "lm_head")
    check(y[M - 1:M], ref, tol, "prefill last row")


# ------------------------------------------------------------------ full sizes, sampled

def _full_cases():
    out = []
    for cfg in (2, 3, 4, 5):
        for i, g in enumerate(synth.CONFIGS[cfg]):
            out.append(pytest.param(g, id=f"config{cfg}_{g.name}"))
    return out


@pytest.mark.parametrize("g", _full_cases())
def test_full_size_sampled(g):
    W = synth.make_weights(g)
    x = synth.make_acts(g)
    y = gpu_prefill(W, g.fmt, x, g.N)
    rng = np.random.default_rng(g.w_seed)
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.integers(0, g.M, 6)]))
    cols = np.unique(np.concatenate([[0, g.N - 1], rng.integers(0, g.N, 96)]))
    ref = oracle.gemm(g.fmt, W, x, g.N, rows=rows, cols=cols)
    tol = bound(x, rows, max_abs_w(g.fmt, W, g.N, g.K))
    r = check(y[np.ix_(rows, cols)], ref, tol, g.name)
    print(f"{g.name}: max err/tol {r:.2e}")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID.get)
@pytest.mark.parametrize("K", [256, 512, 1024, 2048, 2560, 4096, 4352, 6144, 8192, 12288])
@pytest.mark.parametrize("N", [77, 80])
def test_skinny_all_row_splits(fmt, K, N):
    """Skinny path over K values whose super-block counts select every work split
    (several rows per wavefront step, one row per step, several steps per row,
    partial last step) and over M rows whose activations sit in registers, in LDS
    whole, or in LDS one slice of K at a time;
    N = 80 makes every Q6_K matrix a whole number of 16-byte chunks, so the
    coalesced loads run wherever the steps are aligned and K <= 4096 (N = 77
    only for K = 2048 and 4096)."""
    W = synth.pack(fmt, synth.normal(590 + K, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    for M in (1, 2, 5, 8):
        x = synth.to_bf16_bits(synth.normal(591 + M, (M, K)))
        ref = oracle.gemm(fmt, W, x, N)
        tol = bound(x, np.arange(M), wmax)
        check(gpu_prefill(W, fmt, x, N, qg.QG_PATH_SKINNY), ref, tol,
              f"skinny M={M} N={N} K={K} {qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_SKINNY)}")


@pytest.mark.parametrize("fmt", [qg.QG_Q4_K, qg.QG_Q6_K], ids=FMT_ID.get)
def test_skinny_slices_many_rows(fmt):
    """The skinny path with the activations staged one 4096-value slice of K
    at a time (rows too long for the whole of them in LDS): 8300 rows, so
    every wavefront carries several chunks of rows through the slices, and
    K = 8448, whose last slice holds one super-block."""
    N, K = 8300, 8448
    W = synth.pack(fmt, synth.normal(660 + fmt, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    for M in (7, 8):
        name = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_SKINNY)
        assert name == f"skinny_kernel<{fmt}, {M}, 1, 2, 0, 256>", name
        x = synth.to_bf16_bits(synth.normal(661 + M, (M, K)))
        ref = oracle.gemm(fmt, W, x, N)
        check(gpu_prefill(W, fmt, x, N, qg.QG_PATH_SKINNY), ref, bound(x, np.arange(M), wmax),
              f"skinny slices M={M} N={N} K={K} {name}")


# (fmt, K, N, {M: threads per workgroup}): every launch plan of the skinny
# kernel, over weight-row counts that leave some wavefronts a row more than
# others (or, at 8192, none)
SKINNY_PLANS = [
    (qg.QG_Q6_K, 12288, 4100, {2: 1024, 4: 1024, 5: 256}),  # rows in LDS; slices, N % 4096 != 0
    (qg.QG_Q4_K, 9728, 2050, {2: 1024, 5: 1024, 6: 256}),
    (qg.QG_Q6_K, 8448, 8192, {6: 1024, 8: 512}),            # rows in LDS; slices over 2 x 4096 rows
    (qg.QG_Q4_K, 2560, 8197, {1: 256, 3: 512, 6: 512}),     # registers; rows of K <= 4096 in LDS
    (qg.QG_Q6_K, 4096, 2561, {1: 256, 2: 256, 3: 256}),     # field loads (no coalesced loads); LDS
    (qg.QG_Q6_K, 4096, 16400, {5: 512, 8: 512}),            # coalesced loads through registers, 512
    (qg.QG_Q6_K, 2560, 20000, {5: 256, 8: 256}),            # unaligned steps: field loads, 256
]


@pytest.mark.parametrize("fmt,K,N,plans", SKINNY_PLANS,
                         ids=[f"{FMT_ID[f]}-{k}to{n}" for f, k, n, _ in SKINNY_PLANS])
def test_skinny_launch_plans(fmt, K, N, plans):
    """The skinny kernel in each workgroup size and count it launches with
    (1024 threads, one workgroup per CU; 512 threads, two; 256 threads, two
    or more) against the oracle on sampled weight rows that include the last
    ones, which the wavefronts with one row more than the rest compute."""
    W = synth.pack(fmt, synth.normal(700 + K + N, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    rng = np.random.default_rng(K * N)
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(N - 40, N), rng.integers(0, N, 40)]))
    for M, th in plans.items():
        name = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_SKINNY)
        assert name.endswith(f", {th}>"), name
        if fmt == qg.QG_Q6_K and K == 4096 and M <= 2:
            assert name == f"skinny_kernel<1, {M}, 1, 0, 0, 256>", name  # field loads
        x = synth.to_bf16_bits(synth.normal(701 + M, (M, K)))
        y = gpu_prefill(W, fmt, x, N, qg.QG_PATH_SKINNY)
        ref = oracle.gemm(fmt, W, x, N, cols=cols)
        check(y[:, cols], ref, bound(x, np.arange(M), wmax), f"skinny plan M={M} N={N} K={K} {name}")


def test_lm_head_decode_batches():
    """The LM head's full shape (4096 -> 152064 Q6_K) at M = 3, 4 and 6, between
    the workload's M = 1 and 8: the register-staged skinny kernel in 256-thread
    workgroups capped at what a CU holds (three per CU at M = 3 and 4) and in
    one 512-thread workgroup per CU (M = 6), on sampled weight rows that
    include the last ones."""
    g = synth.CONFIGS[5][1]
    assert g.M == 8 and g.N == 152064, g
    W = synth.make_weights(g)
    x8 = synth.make_acts(g)
    wmax = max_abs_w(g.fmt, W, g.N, g.K)
    rng = np.random.default_rng(g.w_seed + 3)
    cols = np.unique(np.concatenate([[0, g.N - 1], np.arange(g.N - 64, g.N), rng.integers(0, g.N, 96)]))
    for M in (3, 4, 6):
        x = np.ascontiguousarray(x8[:M])
        name = qg.qgemm_kernel_name(g.fmt, M, g.N, g.K)
        assert name == f"skinny_kernel<1, {M}, 1, 0, 1, {512 if M >= 5 else 256}>", name
        y = gpu_prefill(W, g.fmt, x, g.N)
        ref = oracle.gemm(g.fmt, W, x, g.N, cols=cols)
        check(y[:, cols], ref, bound(x, np.arange(M), wmax), f"lm head M={M} {name}")


@pytest.mark.parametrize("fmt", [qg.QG_Q4_K, qg.QG_Q5_K], ids=FMT_ID.get)
@pytest.mark.parametrize("N,K", [(700, 256), (16400, 1024), (300, 1024), (300, 2816)])
def test_small_grid_decode_rows(fmt, N, K):
    """The small-grid kernel on decode-sized batches through the tiled path:
    M <= 8 takes the variant that applies the epilogue to the four accumulator
    elements per lane that hold output rows (and loads no other activation
    rows), M = 9 the full one; ragged N, K split over 1, 2, 4 and 8 waves."""
    W = synth.pack(fmt, synth.normal(640 + K, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    for M in (1, 3, 4, 5, 8, 9):
        name = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_TILED)
        assert "_small_kernel<" in name and name.endswith(", 4>" if M <= 8 else ", 16>"), name
        x = synth.to_bf16_bits(synth.normal(641 + M, (M, K)))
        ref = oracle.gemm(fmt, W, x, N)
        check(gpu_prefill(W, fmt, x, N, qg.QG_PATH_TILED), ref, bound(x, np.arange(M), wmax),
              f"small grid M={M} N={N} K={K} {name}")


DECODE_SHAPES = [(1024, 4096), (1024, 7168), (3584, 1024), (2560, 9728), (9728, 2560), (4096, 24576)]


DECODE_CASES = ([(f, k, n) for f in (qg.QG_Q4_K, qg.QG_Q5_K, qg.QG_Q8_0) for k, n in DECODE_SHAPES]
                + [(qg.QG_Q6_K, 4096, 2560), (qg.QG_Q6_K, 12288, 4096)])


@pytest.mark.parametrize("fmt,K,N", DECODE_CASES, ids=[f"{FMT_ID[f]}-{k}to{n}" for f, k, n in DECODE_CASES])
def test_decode_shapes_auto_path(fmt, K, N):
    """The automatic path at the decode projections' real shapes, M = 1..8,
    against the oracle on sampled weight rows that include the first and last
    ones.  Q4_K and Q5_K: the skinny kernel up to the shape's row count, the
    small-grid kernel above it (each side of the switch in every shape); Q6_K
    and Q8_0: the skinny kernel throughout, its activations in registers, whole
    in LDS or one K slice at a time as M and K select."""
    W = synth.pack(fmt, synth.normal(680 + K + N, (N, K), 0.0, 0.02))
    wmax = max_abs_w(fmt, W, N, K)
    x8 = synth.to_bf16_bits(synth.normal(681 + K, (8, K)))
    rng = np.random.default_rng(K + N)
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(N - 8, N), rng.integers(0, N, 40)]))
    kinds = set()
    for M in range(1, 9):
        x = np.ascontiguousarray(x8[:M])
        name = qg.qgemm_kernel_name(fmt, M, N, K)
        kinds.add(name.split("<")[0])
        y = gpu_prefill(W, fmt, x, N)
        ref = oracle.gemm(fmt, W, x, N, cols=cols)
        check(y[:, cols], ref, bound(x, np.arange(M), wmax), f"decode M={M} N={N} K={K} {name}")
    assert "skinny_kernel" in kinds, kinds


@pytest.mark.parametrize("M,N,K", [(500, 20500, 768), (256, 45000, 512)])
def test_mixed_blocks(M, N, K):
    """The mixed-block launch (one round of 128x256 blocks, then 64x256 blocks
    over the remaining columns), ragged in M and in the last column tile: against
    the oracle on sampled rows x columns on both sides of the column split, and
    bit for bit against the one-tile kernel, which a shorter batch of the same
    rows runs (every output element adds its blocks in K order either way)."""
    assert qg.qgemm_kernel_name(qg.QG_Q4_K, M, N, K) == "gemm_q4k_mix_kernel"
    W = synth.pack(qg.QG_Q4_K, synth.normal(690 + K, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(691 + M, (M, K)))
    y = gpu_prefill(W, qg.QG_Q4_K, x, N)
    n1 = 256 * (256 // ((M + 127) // 128))  # the column split
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(M - 5, M), rng.integers(0, M, 10)]))
    cols = np.unique(np.concatenate([[0, n1 - 1, n1, N - 1], np.arange(N - 6, N), rng.integers(0, N, 40)]))
    ref = oracle.gemm(qg.QG_Q4_K, W, x, N, rows=rows, cols=cols)
    check(y[np.ix_(rows, cols)], ref, bound(x, rows, max_abs_w(qg.QG_Q4_K, W, N, K)), f"mixed {M}x{N}x{K}")
    mm = 192 if M > 256 else 100
    short = qg.qgemm_kernel_name(qg.QG_Q4_K, mm, N, K)
    assert short != "gemm_q4k_mix_kernel", short
    assert np.array_equal(y[:mm], gpu_prefill(W, qg.QG_Q4_K, np.ascontiguousarray(x[:mm]), N)), short


@pytest.mark.parametrize("fmt,M,N,K", [
    (qg.QG_Q4_K, 2049, 15300, 1024),   # 128x256 tiles, ragged M and N
    (qg.QG_Q4_K, 4096, 2560, 1024),    # one round of 128x256 blocks, then 128 64x256 blocks (mixed launch)
    (qg.QG_Q4_K, 577, 8240, 768),      # 64x128 tiles at 4 waves/SIMD, ragged (650 blocks: grid order)
    (qg.QG_Q4_K, 577, 8100, 768),      # the same with 640 blocks: the XCD-aware tile order
    (qg.QG_Q4_K, 1000, 2500, 768),     # 64x128 tiles, the grid cut into an 8x5-tile sub-grid per XCD (a = 2), ragged
    (qg.QG_Q4_K, 500, 2500, 1280),     # the same with two K-groups (a = 2), ragged
    (qg.QG_Q4_K, 330, 2700, 1280),     # 64x128 blocks, K split over 2 groups (2 + 3 super-blocks)
    (qg.QG_Q4_K, 170, 2800, 2816),     # 32x64 blocks, K split over 4 groups (2 + 3 + 3 + 3)
    (qg.QG_Q6_K, 2000, 4000, 512),     # one-stage 128x128 tiles (512 blocks: whole rounds), ragged
    (qg.QG_Q6_K, 1100, 8300, 1280),    # half-stage 64x64 blocks (585 128x128 blocks: a ragged round)
    (qg.QG_Q6_K, 600, 8300, 512),      # half-stage 64x64 blocks, ragged
    (qg.QG_Q6_K, 300, 8300, 512),      # half-stage 64x64 blocks
    (qg.QG_Q6_K, 70, 300, 768),        # half-stage 64x64 blocks, K split over 2 groups (1 + 2 super-blocks)
    (qg.QG_Q6_K, 70, 300, 256),        # half-stage 64x64 blocks, one super-block
    (qg.QG_Q4_K, 65, 230, 2048),       # one 32x32 tile per wave, K split over 8 waves
    (qg.QG_Q4_K, 100, 200, 512),       # K split over 2 waves
    (qg.QG_Q5_K, 2049, 16480, 1024),   # Q5_K: 64x128 tiles (the 128x256 pick), ragged
    (qg.QG_Q5_K, 577, 8240, 768),      # 64x128 tiles, ragged
    (qg.QG_Q5_K, 330, 2700, 1280),     # 32x64 blocks, K split over 3 groups (1 + 2 + 2)
    (qg.QG_Q5_K, 170, 2800, 2816),     # 32x64 blocks, K split over 3 groups (3 + 4 + 4)
    (qg.QG_Q5_K, 65, 230, 2048),       # one 32x32 tile per wave, K split over 8 waves
    (qg.QG_Q5_K, 100, 200, 512),       # K split over 2 waves
    (qg.QG_Q8_0, 2049, 15300, 1024),   # Q8_0: 64x128 tiles, ragged
    (qg.QG_Q8_0, 330, 2700, 1280),     # 32x64 blocks, K split over 3 groups
    (qg.QG_Q8_0, 65, 230, 512),        # 32x64 blocks, one K-group (two super-block lengths)
])
def test_tiled_configs_ragged(fmt, M, N, K):
    """Every tiled kernel configuration the dispatcher can pick, on shapes whose
    M and N are not multiples of the tile: sampled rows and columns, always
    including the last row and column and the tile edges around them."""
    W = synth.pack(fmt, synth.normal(600 + M, (N, K), 0.0, 0.02))
    x = synth.to_bf16_bits(synth.normal(601 + N, (M, K)))
    name = qg.qgemm_kernel_name(fmt, M, N, K, qg.QG_PATH_TILED)
    y = gpu_prefill(W, fmt, x, N, qg.QG_PATH_TILED)
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, 63, 64, 127, 128, M - 2, M - 1], rng.integers(0, M, 8)]))
    rows = rows[rows < M]
    cols = np.unique(np.concatenate([[0, 127, 128, 255, 256, N - 33, N - 2, N - 1], rng.integers(0, N, 64)]))
    cols = cols[cols < N]
    ref = oracle.gemm(fmt, W, x, N, rows=rows, cols=cols)
    tol = bound(x, rows, max_abs_w(fmt, W, N, K))
    check(y[np.ix_(rows, cols)], ref, tol, f"{name} M={M} N={N} K={K}")
