"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each function takes an oracle object (the ``oracle`` package, or an
``oracle.Oracle`` bound to another build of the same source) and raises
AssertionError when the oracle disagrees with what the block format and the
mathematics fix:

  * hand-packed super-blocks whose decoded values are known in closed form
    (tests/golden/*.txt; Q4_K, Q5_K, Q6_K, Q8_0),
  * bit probes: every stored bit changes exactly one decoded field by a power
    of two, and every field receives exactly its width in bits,
  * binary16 values fixed by IEEE 754,
  * quantiser properties that hold for any input (error bound, sign symmetry,
    power-of-two covariance, the extreme element maps to +-127, zero blocks),
  * brute-force fp64 dequantise-then-matmul on tiny shapes,
  * the textbook special case (unit scales, zero mins, integer activations
    whose blocks all reach +-127) where the result is a plain integer matmul,
  * closed-form sums of the worked examples under an all-ones activation row,
  * invariants (row / column selection, exact power-of-two scaling of x),
  * for the dequantise-to-fp16 branch: binary16 rounding against numpy's and
    CPython's own conversions, the worked examples (binary16-exact), the
    rounding chain rebuilt from numpy conversions, brute force and the
    textbook integer case,
  * for the per-256 activation variant: quantiser properties, agreement with
    the per-32 oracle where the two encodings coincide, brute force and the
    textbook integer case,
  * for RMSNorm -> quantiser: closed forms (one nonzero value, constant rows,
    a zero row), numpy's fp64 formula within three fp32 roundings, unit mean
    square, power-of-two and sign covariance, row independence,
  * for SwiGLU: silu written with tanh, its limits, and brute force over the
    stacked gate/up product.

The mutation tests plant plausible mistakes in a copy of oracle.c and require
that at least one of these functions fails for each.
"""
from __future__ import annotations

import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q4_K, Q6_K, Q5_K, Q8_0 = 0, 1, 2, 3


def read_fixture(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def _hex(s: str) -> list[int]:
    return [int(t, 16) for t in s.split()]


def q4k_example_block() -> tuple[np.ndarray, dict]:
    fx = read_fixture("q4k_worked_example.txt")
    b = _hex(fx["bytes_0_15"]) + _hex(fx["qs_chunk_32B_repeated_4x"]) * 4
    assert len(b) == 144
    return np.array(b, np.uint8), fx


def q5k_example_block() -> tuple[np.ndarray, dict]:
    fx = read_fixture("q5k_worked_example.txt")
    b = _hex(fx["bytes_0_15"]) + _hex(fx["qh_32B"]) + _hex(fx["qs_chunk_32B_repeated_4x"]) * 4
    assert len(b) == 176
    return np.array(b, np.uint8), fx


def q80_example_block() -> tuple[np.ndarray, dict]:
    """One 34-byte Q8_0 block (32 values)."""
    fx = read_fixture("q80_worked_example.txt")
    b = _hex(fx["bytes"])
    assert len(b) == 34
    return np.array(b, np.uint8), fx


def q6k_example_block() -> tuple[np.ndarray, dict]:
    fx = read_fixture("q6k_worked_example.txt")
    b = (_hex(fx["ql_chunk_32B_repeated_4x"]) * 4 + _hex(fx["qh_chunk_32B_repeated_2x"]) * 2
         + _hex(fx["scales_16B"]) + [0x00, 0x3C])
    assert len(b) == 210
    return np.array(b, np.uint8), fx


# ------------------------------------------------------------------ binary16

def pin_half(orc):
    # IEEE 754 binary16 encodings with textbook values
    cases = {0x0000: 0.0, 0x3C00: 1.0, 0x3800: 0.5, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x3555: 0.333251953125, 0x7C00: float("inf"), 0xFC00: float("-inf")}
    for h, v in cases.items():
        got = orc.half_to_double(h)
        assert got == v, (hex(h), got, v)


# ------------------------------------------------------------------ decoders

def pin_q4k_worked_example(orc):
    blk, fx = q4k_example_block()
    q, sc, m, d, dmin = orc.decode_q4k(blk, 1, 256)
    assert d[0, 0] == 1.0 and dmin[0, 0] == 0.5, (d, dmin)
    assert list(sc[0]) == [int(t) for t in fx["sc"].split()], sc
    assert list(m[0]) == [int(t) for t in fx["m"].split()], m
    v = np.arange(256)
    expect_q = np.where((v // 32) % 2 == 0, v % 16, 15 - v % 16)
    assert np.array_equal(q[0].astype(int), expect_q)
    w = orc.dequant(Q4_K, blk, 1, 256)[0]
    assert w.sum() == float(fx["sum_w"]) and w.min() == float(fx["min_w"]) and w.max() == float(fx["max_w"])


def pin_q5k_worked_example(orc):
    blk, fx = q5k_example_block()
    q, sc, m, d, dmin = orc.decode_q5k(blk, 1, 256)
    assert d[0, 0] == 1.0 and dmin[0, 0] == 0.5, (d, dmin)
    assert list(sc[0]) == [int(t) for t in fx["sc"].split()], sc
    assert list(m[0]) == [int(t) for t in fx["m"].split()], m
    v = np.arange(256)
    j, l = v // 32, v % 32
    low = np.where(j % 2 == 0, v % 16, 15 - v % 16)
    expect_q = low + 16 * ((l >> j) & 1)
    assert np.array_equal(q[0].astype(int), expect_q)
    w = orc.dequant(Q5_K, blk, 1, 256)[0]
    assert w.sum() == float(fx["sum_w"]) and w.min() == float(fx["min_w"]) and w.max() == float(fx["max_w"])


def pin_q80_worked_example(orc):
    blk, fx = q80_example_block()
    q, d = orc.decode_q80(blk, 1, 32)
    assert d[0, 0] == 0.5 and np.array_equal(q[0].astype(int), np.arange(32) - 16)
    blk8 = np.tile(blk, 8)                              # eight blocks: one 256-value row
    w = orc.dequant(Q8_0, blk8, 1, 256)[0]
    assert w[:32].sum() == float(fx["sum_w"]) and w.min() == float(fx["min_w"]) and w.max() == float(fx["max_w"])
    assert np.array_equal(w, np.tile(w[:32], 8))


def pin_q6k_worked_example(orc):
    blk, fx = q6k_example_block()
    q6, sc, d = orc.decode_q6k(blk, 1, 256)
    assert d[0, 0] == 1.0
    assert list(sc[0]) == [int(t) for t in fx["sc"].split()]
    v = np.arange(256)
    quarter = (v % 128) // 32
    expect = np.where(quarter < 2, v % 64, 63 - v % 64)
    assert np.array_equal(q6[0].astype(int), expect)
    w = orc.dequant(Q6_K, blk, 1, 256)[0]
    assert w.sum() == float(fx["sum_w"]) and w.min() == float(fx["min_w"]) and w.max() == float(fx["max_w"])


def _fields_q4k(orc, blk):
    q, sc, m, d, dmin = orc.decode_q4k(blk, 1, 256)
    return {"q": q[0].astype(np.int64), "sc": sc[0].astype(np.int64), "m": m[0].astype(np.int64),
            "d": d[0], "dmin": dmin[0]}


def _fields_q5k(orc, blk):
    q, sc, m, d, dmin = orc.decode_q5k(blk, 1, 256)
    return {"q": q[0].astype(np.int64), "sc": sc[0].astype(np.int64), "m": m[0].astype(np.int64),
            "d": d[0], "dmin": dmin[0]}


def _fields_q80(orc, blk):
    q, d = orc.decode_q80(blk, 1, 32)
    return {"q": q[0].astype(np.int64), "d": d[0]}


def _fields_q6k(orc, blk):
    q6, sc, d = orc.decode_q6k(blk, 1, 256)
    return {"q": q6[0].astype(np.int64), "sc": sc[0].astype(np.int64), "d": d[0]}


def _bit_probe(orc, blk, nbytes, fields_fn, widths, half_fields):
    """Flip every bit: exactly one integer field element changes by +-2^k, or exactly
    one binary16 field changes to the value of the flipped pattern.  Each integer
    field element must receive exactly `width` distinct bit positions 0..width-1."""
    base = fields_fn(orc, blk)
    hits = {name: [set() for _ in range(len(base[name]))] for name in widths}
    half_hits = {name: 0 for name in half_fields}
    for byte in range(nbytes):
        for bit in range(8):
            b2 = blk.copy()
            b2[byte] ^= np.uint8(1 << bit)
            f2 = fields_fn(orc, b2)
            changed = []
            for name in widths:
                idx = np.nonzero(f2[name] != base[name])[0]
                for i in idx:
                    changed.append((name, int(i), int(f2[name][i] - base[name][i])))
            for name, off in half_fields.items():
                if f2[name][0] != base[name][0]:
                    h = int(b2[off]) | (int(b2[off + 1]) << 8)
                    assert f2[name][0] == orc.half_to_double(h), (byte, bit, name)
                    changed.append((name, 0, None))
            assert len(changed) == 1, (byte, bit, changed)
            name, i, delta = changed[0]
            if name in half_fields:
                half_hits[name] += 1
                continue
            k = int(np.log2(abs(delta)))
            assert abs(delta) == 1 << k, (byte, bit, delta)
            assert k not in hits[name][i], (byte, bit, name, i, k)
            hits[name][i].add(k)
    for name, w in widths.items():
        for i, s in enumerate(hits[name]):
            assert s == set(range(w)), (name, i, s)
    for name in half_fields:
        assert half_hits[name] == 16, (name, half_hits[name])


def pin_q4k_bit_probe(orc):
    blk = synth.random_blocks(Q4_K, 1, 256, seed=77, emin=1, emax=14, allow_negative=False)[0]
    _bit_probe(orc, blk, 144, _fields_q4k, {"q": 4, "sc": 6, "m": 6}, {"d": 0, "dmin": 2})


def pin_q5k_bit_probe(orc):
    blk = synth.random_blocks(Q5_K, 1, 256, seed=79, emin=1, emax=14, allow_negative=False)[0]
    _bit_probe(orc, blk, 176, _fields_q5k, {"q": 5, "sc": 6, "m": 6}, {"d": 0, "dmin": 2})


def pin_q80_bit_probe(orc):
    blk = synth.random_blocks(Q8_0, 1, 256, seed=80, emin=1, emax=14, allow_negative=False)[0][:34]
    _bit_probe(orc, blk.copy(), 34, _fields_q80, {"q": 8}, {"d": 0})


def pin_q6k_bit_probe(orc):
    blk = synth.random_blocks(Q6_K, 1, 256, seed=78, emin=1, emax=14, allow_negative=False)[0]
    _bit_probe(orc, blk, 210, _fields_q6k, {"q": 6, "sc": 8}, {"d": 208})


# ------------------------------------------------------------------ quantiser

def _acts(seed, M, K, scale=1.0):
    x = synth.normal(seed, (M, K)) * np.float32(scale)
    return x.astype(np.float32)


def pin_quant_all_ones(orc):
    fx = read_fixture("q4k_worked_example.txt")
    x = np.ones((1, 256), np.float32)
    q, d, S = orc.quantize_act(x)
    assert np.all(q == 127) and np.all(S == 4064)
    assert np.all(d == np.float32(float(fx["dx_all_ones"])))


def pin_quant_zero_block(orc):
    x = _acts(5, 2, 128)
    x[1, 32:64] = 0.0
    x[0, :32] = -0.0
    q, d, S = orc.quantize_act(x)
    assert d[1, 1] == 0.0 and S[1, 1] == 0 and np.all(q[1, 32:64] == 0)
    assert d[0, 0] == 0.0 and np.all(q[0, :32] == 0)
    assert np.all(d[0, 1:] > 0)


def pin_quant_properties(orc):
    x = _acts(11, 8, 1024)
    x[3, :] *= np.float32(1e-30)          # tiny but normal
    x[4, 100] = np.float32(37.0)          # outlier
    x[5, ::7] = 0.0                       # scattered zeros
    q, d, S = orc.quantize_act(x)
    M, K = x.shape
    qb = q.reshape(M, K // 32, 32).astype(np.int64)
    xb = x.reshape(M, K // 32, 32).astype(np.float64)
    db = d.astype(np.float64)[:, :, None]
    assert np.all(np.abs(qb) <= 127)
    assert np.array_equal(S, qb.sum(-1).astype(np.int32))
    # the extreme element of every block maps to +-127
    amax = np.abs(xb).max(-1)
    imax = np.abs(xb).argmax(-1)
    qmax = np.take_along_axis(qb, imax[:, :, None], -1)[:, :, 0]
    assert np.all(np.abs(qmax) == 127)
    # d is amax/127 correctly rounded to fp32: |d*127 - amax| <= 127 * ulp(d)/2
    ulp = np.spacing(d.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(d.astype(np.float64) * 127 - amax) <= 127 * ulp / 2 * 1.0000001)
    # reconstruction error: |x - d*q| <= d/2 (plus the rounding of 1/d and x*id)
    err = np.abs(xb - db * qb)
    assert np.all(err <= db * 0.50002), err.max()
    # zero maps to zero
    assert np.all(q[5, ::7] == 0)


def pin_quant_symmetry_and_scaling(orc):
    x = _acts(12, 4, 512)
    q, d, S = orc.quantize_act(x)
    qn, dn, Sn = orc.quantize_act(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d) and np.array_equal(Sn, -S)
    for k in (-20, -3, 1, 7):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        qs, ds, Ss = orc.quantize_act(xs)
        assert np.array_equal(qs, q) and np.array_equal(Ss, S)
        assert np.array_equal(ds, (d * np.float32(2.0 ** k)).astype(np.float32))


def pin_quant_integer_blocks(orc):
    # blocks of integers in [-127, 127] that contain +-127 quantise to themselves with d = 1
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, size=(3, 256))
    xi[:, ::32] = 127 * np.where(rng.random((3, 8)) < 0.5, -1, 1)
    q, d, S = orc.quantize_act(xi.astype(np.float32))
    assert np.all(d == 1.0) and np.array_equal(q.astype(np.int64), xi)
    # with d = 1 exactly, half-integers are ties: IEEE round-half-to-even decides them
    xh = np.zeros((1, 32), np.float32)
    xh[0, :9] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -3.5]
    q, d, _ = orc.quantize_act(xh)
    assert d[0, 0] == 1.0
    assert list(q[0, :9]) == [127, 0, 2, 2, 0, -2, -2, 126, -4], q[0, :9]


def pin_quant_bf16_matches_f32(orc):
    xb = synth.to_bf16_bits(_acts(13, 4, 256))
    xf = synth.bf16_bits_to_f32(xb)
    a = orc.quantize_act(xb)
    b = orc.quantize_act(xf)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------------------------------ GEMM

def _dequant_acts(orc, x):
    q, d, S = orc.quantize_act(x)
    M, K = q.shape
    return (q.reshape(M, K // 32, 32).astype(np.float64) * d.astype(np.float64)[:, :, None]).reshape(M, K)


def _bruteforce_case(orc, fmt, W, x, N):
    y = orc.gemm(fmt, W, x, N)
    w = orc.dequant(fmt, W, N, x.shape[1])
    xh = _dequant_acts(orc, x)
    ref = xh @ w.T
    scale = np.abs(xh) @ np.abs(w).T + 1e-300
    assert np.all(np.abs(y - ref) <= 1e-12 * scale), np.max(np.abs(y - ref) / scale)


def pin_gemm_bruteforce(orc):
    for fmt in (Q4_K, Q5_K, Q6_K, Q8_0):
        for (M, N, K, seed) in ((1, 1, 256, 1), (3, 5, 256, 2), (4, 8, 512, 3), (2, 7, 768, 4)):
            Wr = synth.random_blocks(fmt, N, K, seed=100 + seed, emin=3, emax=18)
            Wp = synth.pack(fmt, synth.normal(200 + seed, (N, K), 0.0, 0.02))
            x = _acts(300 + seed, M, K)
            _bruteforce_case(orc, fmt, Wr, x, N)
            _bruteforce_case(orc, fmt, Wp, synth.to_bf16_bits(x), N)


def _textbook_blocks(fmt, N, K, seed):
    """Blocks with unit scales and zero mins and random codes, plus those codes."""
    rng = np.random.default_rng(seed)
    nb = K // 256
    if fmt == Q4_K:
        W = np.zeros((N, nb, 144), np.uint8)
        W[:, :, 0:2] = (0x00, 0x3C)              # d = 1
        W[:, :, 2:4] = (0x00, 0x00)              # dmin = 0
        W[:, :, 4:8] = 1                         # sc[0..3] = 1, top bits 0
        W[:, :, 8:12] = 0                        # m[0..3] = 0
        W[:, :, 12:16] = 0x01                    # sc[4..7] = 1, m[4..7] = 0
        codes = rng.integers(0, 16, size=(N, nb, 256))
        for v in range(256):
            byte = 16 + 32 * (v // 64) + v % 32
            shift = 0 if v % 64 < 32 else 4
            W[:, :, byte] |= (codes[:, :, v] << shift).astype(np.uint8)
        vals = codes
    elif fmt == Q8_0:
        W = np.zeros((N, nb, 8, 34), np.uint8)
        W[:, :, :, 0:2] = (0x00, 0x3C)           # d = 1 in every 32-value block
        codes = rng.integers(-127, 128, size=(N, nb, 8, 32))
        W[:, :, :, 2:] = codes.astype(np.int8).view(np.uint8)
        vals = codes
    elif fmt == Q5_K:
        W = np.zeros((N, nb, 176), np.uint8)
        W[:, :, 0:2] = (0x00, 0x3C)              # d = 1
        W[:, :, 4:8] = 1                         # sc[0..3] = 1; dmin = 0, m = 0
        W[:, :, 12:16] = 0x01                    # sc[4..7] = 1
        codes = rng.integers(0, 32, size=(N, nb, 256))
        for v in range(256):
            byte = 48 + 32 * (v // 64) + v % 32
            shift = 0 if v % 64 < 32 else 4
            W[:, :, byte] |= ((codes[:, :, v] & 15) << shift).astype(np.uint8)
            W[:, :, 16 + v % 32] |= (((codes[:, :, v] >> 4) & 1) << (v // 32)).astype(np.uint8)
        vals = codes
    else:
        W = np.zeros((N, nb, 210), np.uint8)
        W[:, :, 192:208] = 1                     # sc = 1
        W[:, :, 208:210] = (0x00, 0x3C)          # d = 1
        codes = rng.integers(0, 64, size=(N, nb, 256))
        for v in range(256):
            h, r = divmod(v, 128)
            c, l = divmod(r, 32)
            lb = 64 * h + 32 * (c % 2) + l
            W[:, :, lb] |= ((codes[:, :, v] & 15) << (0 if c < 2 else 4)).astype(np.uint8)
            W[:, :, 128 + 32 * h + l] |= (((codes[:, :, v] >> 4) & 3) << (2 * c)).astype(np.uint8)
        vals = codes - 32
    return W.reshape(N, -1), vals.reshape(N, K).astype(np.int64)


def _integer_acts(M, K, seed):
    rng = np.random.default_rng(seed)
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, ::32] = 127 * np.where(rng.random((M, K // 32)) < 0.5, -1, 1)
    return xi


def pin_gemm_textbook(orc):
    for fmt in (Q4_K, Q5_K, Q6_K, Q8_0):
        M, N, K = 5, 6, 512
        W, wv = _textbook_blocks(fmt, N, K, seed=9 + fmt)
        xi = _integer_acts(M, K, seed=19 + fmt)
        y = orc.gemm(fmt, W, xi.astype(np.float32), N)
        exact = xi @ wv.T                          # int64 textbook matmul
        assert np.array_equal(y, exact.astype(np.float64)), np.abs(y - exact).max()
        # per-block integer partials are block-wise textbook matmuls
        L = 16 if fmt == Q6_K else 32
        P = orc.block_partials(fmt, W, xi.astype(np.int8), N)
        ref = np.einsum("mbt,nbt->mnb", xi.reshape(M, K // L, L), wv.reshape(N, K // L, L))
        assert np.array_equal(P.astype(np.int64), ref)


def pin_gemm_worked_examples(orc):
    x = np.ones((1, 256), np.float32)
    dx = np.float64(np.float32(1.0) / np.float32(127.0))
    blk4, fx4 = q4k_example_block()
    y4 = orc.gemm(Q4_K, blk4, x, 1)[0, 0]
    assert abs(y4 - float(fx4["sum_w"]) * 127 * dx) <= 1e-9, y4
    blk5, fx5 = q5k_example_block()
    y5 = orc.gemm(Q5_K, blk5, x, 1)[0, 0]
    assert abs(y5 - float(fx5["sum_w"]) * 127 * dx) <= 1e-9, y5
    blk8, fx8 = q80_example_block()
    y8 = orc.gemm(Q8_0, np.tile(blk8, 8), x, 1)[0, 0]
    assert abs(y8 - 8 * float(fx8["sum_w"]) * 127 * dx) <= 1e-12, y8
    blk6, fx6 = q6k_example_block()
    y6 = orc.gemm(Q6_K, blk6, x, 1)[0, 0]
    assert abs(y6 - float(fx6["sum_w"]) * 127 * dx) <= 1e-12, y6


def pin_gemm_selection_and_scaling(orc):
    for fmt in (Q4_K, Q5_K, Q6_K, Q8_0):
        M, N, K = 6, 9, 512
        W = synth.pack(fmt, synth.normal(41 + fmt, (N, K), 0.0, 0.02))
        x = _acts(43 + fmt, M, K)
        y = orc.gemm(fmt, W, x, N)
        rows, cols = np.array([4, 0, 5]), np.array([8, 1, 3, 3])
        ys = orc.gemm(fmt, W, x, N, rows=rows, cols=cols)
        assert np.array_equal(ys, y[np.ix_(rows, cols)])
        # each output row depends only on its own input row
        assert np.array_equal(orc.gemm(fmt, W, x[2:4].copy(), N), y[2:4])
        y2 = orc.gemm(fmt, W, (x * np.float32(8.0)).astype(np.float32), N)
        assert np.array_equal(y2, y * 8.0)


def pin_gemm_semantic_bound(orc):
    """The quantised result stays within the activation-rounding bound of the
    unquantised product (catches a quantiser that only agrees with itself)."""
    for fmt in (Q4_K, Q5_K, Q6_K, Q8_0):
        M, N, K = 4, 6, 768
        W = synth.pack(fmt, synth.normal(51 + fmt, (N, K), 0.0, 0.02))
        x = _acts(53 + fmt, M, K)
        y = orc.gemm(fmt, W, x, N)
        w = orc.dequant(fmt, W, N, K)
        exact = x.astype(np.float64) @ w.T
        _, d, _ = orc.quantize_act(x)
        dk = np.repeat(d.astype(np.float64), 32, axis=1)       # d of the block holding k
        bound = (dk * 0.50002) @ np.abs(w).T
        assert np.all(np.abs(y - exact) <= bound + 1e-12)


# ------------------------------------------------- dequantise-to-fp16 branch

def _np_f16(v) -> np.ndarray:
    """binary16 bits of float64 values, rounded by numpy's own conversion."""
    with np.errstate(over="ignore"):
        return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def pin_f16_rounding(orc):
    """Round-to-nearest-even binary16 from double, against numpy's conversion and
    CPython's struct 'e' packing (two independent implementations)."""
    import struct
    rng = np.random.default_rng(7)
    quanta = 2.0 ** rng.integers(-34, 6, 4000)
    vals = [rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),
            (rng.integers(0, 2048, 4000) + 0.5) * quanta,                    # exact ties
            (rng.integers(0, 2048, 4000) + 0.5) * quanta * (1 + 2.0 ** -40),  # just above a tie
            (rng.integers(0, 2048, 4000) + 0.5) * quanta * (1 - 2.0 ** -40),  # just below a tie
            np.array([0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -26,
                      65504.0, 65519.99, 65520.0, -65520.0, 1e30, -1e-30, 1 + 2.0 ** -11 + 2.0 ** -40])]
    v = np.concatenate(vals)
    got = np.array([orc.f64_to_f16(t) for t in v], np.uint16)
    assert np.array_equal(got, _np_f16(v)), v[got != _np_f16(v)][:5]
    for t in v[np.abs(v) < 65520][:3000]:
        assert orc.f64_to_f16(t) == struct.unpack("<H", struct.pack("<e", t))[0], t


def pin_f16_activations(orc):
    x = _acts(61, 3, 512, scale=3.0)
    x[0, :7] = [0.0, -0.0, 1e-9, -7e-6, 65519.0, 6e-5, -2.5]
    assert np.array_equal(orc.x_to_f16(x), _np_f16(x.astype(np.float64)))
    b = synth.to_bf16_bits(x)
    assert np.array_equal(orc.x_to_f16(b), _np_f16(synth.bf16_bits_to_f32(b).astype(np.float64)))


def _np_dequant_f16(orc, fmt, W, N, K):
    """The fp16 rounding chain written with numpy conversions, on fields decoded
    by the (separately pinned) block decoders.  A zero weight is compared as +0
    (its sign is not part of the method)."""
    if fmt == Q4_K:
        q, sc, m, d, dmin = orc.decode_q4k(W, N, K)
        d32 = np.repeat(d, 8, axis=1)
        dm32 = np.repeat(dmin, 8, axis=1)
        dsc = _np_f16(d32 * sc).view(np.float16).astype(np.float64)
        dmn = _np_f16(dm32 * m).view(np.float16).astype(np.float64)
        exact = np.repeat(dsc, 32, axis=1) * q - np.repeat(dmn, 32, axis=1)
    else:
        q6, sc, d = orc.decode_q6k(W, N, K)
        dsc = _np_f16(np.repeat(d, 16, axis=1) * sc).view(np.float16).astype(np.float64)
        exact = np.repeat(dsc, 16, axis=1) * (q6.astype(np.float64) - 32)
    return _np_f16(exact + 0.0)


def pin_f16_dequant_worked_examples(orc):
    blk4, fx4 = q4k_example_block()
    w4 = orc.dequant_f16(Q4_K, blk4, 1, 256).view(np.float16).astype(np.float64)
    assert w4.sum() == float(fx4["sum_w"])                     # every value is binary16-exact
    assert w4.min() == float(fx4["min_w"]) and w4.max() == float(fx4["max_w"])
    blk6, fx6 = q6k_example_block()
    w6 = orc.dequant_f16(Q6_K, blk6, 1, 256).view(np.float16).astype(np.float64)
    assert w6.sum() == float(fx6["sum_w"])


def pin_f16_dequant_rounding(orc):
    for fmt in (Q4_K, Q6_K):
        # exponents up to 23: every d*sc stays below 65504, so the rounded
        # sub-block scales are finite (scales that overflow are outside the domain)
        for seed, (emin, emax) in ((3, (1, 23)), (4, (10, 20)), (5, (1, 6))):
            N, K = 9, 512
            W = synth.random_blocks(fmt, N, K, seed=700 + seed, emin=emin, emax=emax)
            assert np.array_equal(orc.dequant_f16(fmt, W, N, K), _np_dequant_f16(orc, fmt, W, N, K))
    # a hand-built case: d = 1 + 2^-10 and sc = 3 give d*sc = 3 + 3*2^-10, a binary16 tie
    # between 3 + 2^-9 and 3 + 2^-8 that goes to the even 3 + 2^-8
    blk = np.zeros(144, np.uint8)
    blk[0:2] = (0x01, 0x3C)
    blk[4] = 3
    blk[16] = 0x01                                                # q[0] = 1
    w = orc.dequant_f16(Q4_K, blk, 1, 256).view(np.float16).astype(np.float64)
    assert w[0, 0] == 3 + 2.0 ** -8 and w[0, 1] == 0.0


def pin_f16_gemm_bruteforce(orc):
    for fmt in (Q4_K, Q6_K):
        for (M, N, K, seed) in ((1, 1, 256, 1), (3, 5, 512, 2), (4, 7, 768, 3)):
            W = synth.random_blocks(fmt, N, K, seed=800 + seed, emin=5, emax=18)
            x = _acts(900 + seed, M, K)
            for xin in (x, synth.to_bf16_bits(x)):
                y, ya = orc.gemm_deq_f16(fmt, W, xin, N)
                xf = x.astype(np.float64) if xin.dtype == np.float32 else \
                    synth.bf16_bits_to_f32(xin).astype(np.float64)
                x16 = _np_f16(xf).view(np.float16).astype(np.float64)
                w16 = _np_dequant_f16(orc, fmt, W, N, K).view(np.float16).astype(np.float64)
                ref, refabs = x16 @ w16.T, np.abs(x16) @ np.abs(w16).T
                assert np.all(np.abs(y - ref) <= 1e-12 * refabs + 1e-300)
                assert np.allclose(ya, refabs, rtol=1e-12, atol=0)


def pin_f16_gemm_textbook(orc):
    for fmt in (Q4_K, Q6_K):
        M, N, K = 5, 6, 512
        W, wv = _textbook_blocks(fmt, N, K, seed=29 + fmt)
        xi = _integer_acts(M, K, seed=39 + fmt)
        y, _ = orc.gemm_deq_f16(fmt, W, xi.astype(np.float32), N)
        assert np.array_equal(y, (xi @ wv.T).astype(np.float64))
        rows, cols = np.array([4, 1]), np.array([5, 0, 0])
        ys, _ = orc.gemm_deq_f16(fmt, W, xi.astype(np.float32), N, rows=rows, cols=cols)
        assert np.array_equal(ys, y[np.ix_(rows, cols)])


# ------------------------------------------------- per-256 activation scales

def pin_a256_quantiser_properties(orc):
    x = _acts(71, 6, 1024, scale=2.0)
    x[0, :256] = 0.0                                    # an all-zero super-block
    x[1, 256:512] *= np.float32(2.0 ** -20)             # tiny values
    x[2, 300] = np.float32(-9.0)                        # an extreme element
    q, d, S = orc.quantize_act256(x)
    assert d[0, 0] == 0 and not q[0, :256].any() and not S[0, :8].any()
    xq = q.reshape(6, 4, 256).astype(np.float64) * d.astype(np.float64)[:, :, None]
    err = np.abs(xq.reshape(6, 1024) - x.astype(np.float64))
    assert np.all(err <= 0.50002 * np.repeat(d.astype(np.float64), 256, axis=1))
    amax = np.abs(x.reshape(6, 4, 256)).max(2)
    assert np.array_equal(d, (amax / np.float32(127.0)).astype(np.float32))
    assert q[2, 300] == -127
    assert np.array_equal(S, q.reshape(6, 32, 32).astype(np.int64).sum(2))
    q2, d2, S2 = orc.quantize_act256(-x)
    assert np.array_equal(q2, -q) and np.array_equal(d2, d) and np.array_equal(S2, -S)
    q3, d3, _ = orc.quantize_act256((x * np.float32(8.0)).astype(np.float32))
    assert np.array_equal(q3, q) and np.array_equal(d3, d * np.float32(8.0))


def pin_a256_matches_per32_when_scales_agree(orc):
    """When every 32-value block of a super-block holds the super-block's extreme
    value, the per-32 and per-256 encodings coincide, and so must the GEMMs."""
    M, N, K = 4, 7, 768
    x = _acts(73, M, K)
    x = np.clip(x, -2.5, 2.5).astype(np.float32)
    x[:, ::32] = np.float32(3.0) * np.where(np.arange(K // 32) % 2 == 0, 1, -1).astype(np.float32)
    q, d, S = orc.quantize_act256(x)
    q32, d32, S32 = orc.quantize_act(x)
    assert np.array_equal(q, q32) and np.array_equal(S, S32)
    assert np.array_equal(np.repeat(d, 8, axis=1), d32)
    W = synth.pack(Q4_K, synth.normal(74, (N, K), 0.0, 0.02))
    assert np.array_equal(orc.gemm_a256(W, x, N), orc.gemm(Q4_K, W, x, N))


def pin_a256_gemm_bruteforce(orc):
    for (M, N, K, seed) in ((1, 1, 256, 1), (3, 5, 512, 2), (4, 8, 768, 3)):
        W = synth.random_blocks(Q4_K, N, K, seed=760 + seed, emin=3, emax=18)
        x = _acts(770 + seed, M, K)
        for xin in (x, synth.to_bf16_bits(x)):
            y = orc.gemm_a256(W, xin, N)
            q, d, _ = orc.quantize_act256(xin)
            xh = (q.reshape(M, K // 256, 256).astype(np.float64) * d.astype(np.float64)[:, :, None]).reshape(M, K)
            w = orc.dequant(Q4_K, W, N, K)
            ref, scale = xh @ w.T, np.abs(xh) @ np.abs(w).T + 1e-300
            assert np.all(np.abs(y - ref) <= 1e-12 * scale)


def pin_a256_gemm_textbook(orc):
    M, N, K = 5, 6, 512
    W, wv = _textbook_blocks(Q4_K, N, K, seed=79)
    rng = np.random.default_rng(80)
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, ::256] = 127                                   # every super-block reaches 127: d = 1
    y = orc.gemm_a256(W, xi.astype(np.float32), N)
    assert np.array_equal(y, (xi @ wv.T).astype(np.float64))
    rows, cols = np.array([3, 0]), np.array([5, 2, 2])
    assert np.array_equal(orc.gemm_a256(W, xi.astype(np.float32), N, rows=rows, cols=cols),
                          y[np.ix_(rows, cols)])


# ------------------------------------------- RMSNorm -> quantiser, and SwiGLU

def pin_rms_single_nonzero(orc):
    """One nonzero value a (a power of two) in a row of K = 1024, eps = 0: the
    mean square is a^2/1024, so r = 32/|a| exactly and xn = -32*g there (a < 0),
    0 elsewhere; the quantiser maps that value to -127*sign(g)."""
    K = 1024
    g = synth.normal(901, (K,), 0.0, 1.0).astype(np.float32)
    x = np.zeros((2, K), np.float32)
    x[0, 37] = np.float32(-0.5)
    x[1, 1000] = np.float32(2.0 ** -40)
    r, lo, hi = orc.rms_scale(x, 0.0)
    assert r[0] == 64.0 and r[1] == np.float32(2.0 ** 45)
    assert np.array_equal(lo, r) and np.array_equal(hi, r)
    xn = orc.rmsnorm(x, g, r)
    assert xn[0, 37] == np.float32(-32.0) * g[37] and xn[1, 1000] == np.float32(32.0) * g[1000]
    assert np.count_nonzero(xn[0]) == 1 and np.count_nonzero(xn[1]) == 1
    q, d, S, amb, _ = orc.rmsnorm_quantize(x, g, 0.0)
    assert not amb.any()
    assert q[0, 37] == -127 * np.sign(g[37]) and q[1, 1000] == 127 * np.sign(g[1000])
    assert np.count_nonzero(q) == 2 and S[0, 1] == q[0, 37]


def pin_rms_constant_rows(orc):
    """x = c on the whole row, eps = 0: r = 1/|c| and xn = sign(c)*g (exactly for
    a power of two c, within one fp32 rounding of each of the three steps else)."""
    K = 512
    g = synth.normal(902, (K,), 0.0, 2.0).astype(np.float32)
    cs = np.array([0.25, -8.0, 3.0, -0.7, 1e-20, 1e20], np.float32)
    x = np.repeat(cs[:, None], K, axis=1)
    r, _, _ = orc.rms_scale(x, 0.0)
    xn = orc.rmsnorm(x, g, r).astype(np.float64)
    ref = np.sign(cs.astype(np.float64))[:, None] * g.astype(np.float64)[None, :]
    assert np.array_equal(xn[:2], ref[:2])
    assert np.all(np.abs(xn - ref) <= 4 * 2.0 ** -24 * np.abs(ref))


def pin_rms_zero_row_and_eps(orc):
    """A zero row gives r = f32(1/sqrt(eps)), xn = 0 and all-zero blocks; eps
    enters as v = mean + eps (a row far below eps is scaled by ~1/sqrt(eps))."""
    K, eps = 256, 1e-6
    g = np.full(K, 1.0, np.float32)
    x = np.zeros((2, K), np.float32)
    x[1] = np.float32(1e-9)
    r, _, _ = orc.rms_scale(x, eps)
    e64 = float(np.float32(eps))
    assert r[0] == np.float32(1.0 / np.sqrt(e64))
    assert abs(float(r[1]) - 1.0 / np.sqrt(e64 + float(np.float32(1e-9)) ** 2)) <= 2.0 ** -23 * float(r[1])
    q, d, S, _, _ = orc.rmsnorm_quantize(x, g, eps)
    assert not q[0].any() and not d[0].any() and not S[0].any()
    assert np.all(np.abs(q[1]) == 127)


def pin_rms_against_numpy(orc):
    """Random rows of several lengths (fp32 and bf16 input, with eps): xn within
    three fp32 roundings of x*g/sqrt(mean(x^2)+eps) evaluated by numpy in fp64;
    the normalised rows have unit mean square (eps = 0)."""
    for K, eps, seed in ((256, 1e-6, 903), (1024, 1e-5, 904), (4096, 0.0, 905)):
        x = _acts(seed, 5, K, scale=3.0)
        x[2] *= np.float32(1e-3)
        g = synth.normal(seed + 1, (K,), 1.0, 0.3).astype(np.float32)
        for xin in (x, synth.to_bf16_bits(x)):
            xf = xin if xin.dtype == np.float32 else synth.bf16_bits_to_f32(xin)
            r, lo, hi = orc.rms_scale(xin, eps)
            assert np.all(lo <= r) and np.all(r <= hi)
            xn = orc.rmsnorm(xin, g, r).astype(np.float64)
            x64 = xf.astype(np.float64)
            ref = x64 * g.astype(np.float64) / np.sqrt((x64 ** 2).mean(1, keepdims=True) + float(np.float32(eps)))
            assert np.all(np.abs(xn - ref) <= 3 * 2.0 ** -24 * np.abs(ref) + 1e-300)
            if eps == 0.0:
                ms = ((xn / g.astype(np.float64)) ** 2).mean(1)
                assert np.all(np.abs(ms - 1.0) < 1e-6)


def pin_rms_scale_invariance_and_rows(orc):
    """eps = 0: scaling a row by a power of two leaves xn unchanged and negating
    it negates xn; each row is normalised by its own statistics only."""
    K = 768
    x = _acts(906, 4, K)
    g = synth.normal(907, (K,), 0.0, 1.0).astype(np.float32)
    q, d, S, _, _ = orc.rmsnorm_quantize(x, g, 0.0)
    for k in (-30, 7):
        q2, d2, S2, _, _ = orc.rmsnorm_quantize((x * np.float32(2.0 ** k)).astype(np.float32), g, 0.0)
        assert np.array_equal(q2, q) and np.array_equal(d2, d) and np.array_equal(S2, S)
    q3, d3, S3, _, _ = orc.rmsnorm_quantize(-x, g, 0.0)
    assert np.array_equal(q3, -q) and np.array_equal(d3, d)
    x4 = x.copy()
    x4[1:] *= np.float32(5.0)
    q4, d4, _, _, _ = orc.rmsnorm_quantize(x4, g, 0.0)
    assert np.array_equal(q4[0], q[0]) and np.array_equal(d4[0], d[0])


def pin_rms_order_band(orc):
    """The sum of squares in another order can give another r32: a row of 1000
    small values (each square under a quarter of the big value's spacing) and
    one big value last.  Summed in row order the small squares survive and
    r32 = 1; summed big value first each is rounded away and r32 = 1 + 2^-23.
    Both orders' r32 must lie in the oracle's band."""
    K = 4096
    x = np.zeros((1, K), np.float32)
    x[0, :1000] = np.float32(1.5 * 2.0 ** -22)
    x[0, K - 1] = np.float32(64.0 * (1.0 - 2.0 ** -24))
    r, lo, hi = orc.rms_scale(x, 0.0)
    sq = [float(t) * float(t) for t in x[0]]
    got = []
    for order in (sq, sq[::-1]):
        ss = 0.0
        for t in order:
            ss += t
        got.append(np.float32(1.0 / np.sqrt(ss / K)))
    assert got[0] != got[1]
    assert r[0] == got[0] and lo[0] <= min(got) and max(got) <= hi[0]


def pin_swiglu_closed_forms(orc):
    """silu(z) = z * (1 + tanh(z/2)) / 2 (the logistic function written with
    tanh), silu(0) = 0, silu(z) -> z for large z and -> 0 (no NaN) for very
    negative z."""
    z = np.linspace(-30.0, 30.0, 601)
    u = synth.normal(908, (601,), 0.0, 2.0).astype(np.float64)
    h = orc.swiglu(z, u)
    ref = z * (1.0 + np.tanh(z / 2.0)) / 2.0 * u
    assert np.all(np.abs(h - ref) <= 1e-14 * np.abs(z * u) + 1e-300)
    h = orc.swiglu(np.array([0.0, 800.0, -800.0, 40.0, -1.0]), np.array([5.0, 2.0, 3.0, 1.0, 1.0]))
    assert h[0] == 0.0 and h[1] == 1600.0 and h[2] == 0.0 and h[3] == 40.0
    assert abs(h[4] - (-1.0 / (1.0 + np.e))) <= 1e-16


def pin_gemm_swiglu_bruteforce(orc):
    """SwiGLU over the stacked [gate; up] weight rows: brute force from the
    quantised activations and the dequantised weights in fp64, gate = columns
    0..F-1 and up = F..2F-1 of the stacked product."""
    for fmt, (M, F, K, seed) in ((Q4_K, (3, 5, 512, 1)), (Q6_K, (2, 4, 256, 2))):
        W = synth.random_blocks(fmt, 2 * F, K, seed=910 + seed, emin=3, emax=18)
        x = _acts(920 + seed, M, K, scale=4.0)
        h, g, u = orc.gemm_swiglu(fmt, W, x, F)
        xh = _dequant_acts(orc, x)
        w = orc.dequant(fmt, W, 2 * F, K)
        y = xh @ w.T
        gate, up = y[:, :F], y[:, F:]
        scale = np.abs(xh) @ np.abs(w).T
        assert np.all(np.abs(g - gate) <= 1e-12 * scale[:, :F]) and np.all(np.abs(u - up) <= 1e-12 * scale[:, F:])
        ref = gate * (1.0 + np.tanh(gate / 2.0)) / 2.0 * up
        assert np.all(np.abs(h - ref) <= 1e-9 * (scale[:, :F] * scale[:, F:] + 1e-300))
        rows, cols = np.array([M - 1, 0]), np.array([F - 1, 1, 1])
        hs, _, _ = orc.gemm_swiglu(fmt, W, x, F, rows=rows, cols=cols)
        assert np.array_equal(hs, h[np.ix_(rows, cols)])


ALL_PINS = [pin_half, pin_q4k_worked_example, pin_q6k_worked_example, pin_q4k_bit_probe,
            pin_q6k_bit_probe, pin_q5k_worked_example, pin_q5k_bit_probe, pin_q80_worked_example,
            pin_q80_bit_probe, pin_quant_all_ones, pin_quant_zero_block, pin_quant_properties,
            pin_quant_symmetry_and_scaling, pin_quant_integer_blocks, pin_quant_bf16_matches_f32,
            pin_gemm_bruteforce, pin_gemm_textbook, pin_gemm_worked_examples,
            pin_gemm_selection_and_scaling, pin_gemm_semantic_bound,
            pin_f16_rounding, pin_f16_activations, pin_f16_dequant_worked_examples,
            pin_f16_dequant_rounding, pin_f16_gemm_bruteforce, pin_f16_gemm_textbook,
            pin_a256_quantiser_properties, pin_a256_matches_per32_when_scales_agree,
            pin_a256_gemm_bruteforce, pin_a256_gemm_textbook,
            pin_rms_single_nonzero, pin_rms_constant_rows, pin_rms_zero_row_and_eps,
            pin_rms_against_numpy, pin_rms_scale_invariance_and_rows, pin_rms_order_band,
            pin_swiglu_closed_forms,
            pin_gemm_swiglu_bruteforce]
