"""The seeded input generator: published splitmix64 outputs, regenerable slices,
distribution moments, and legal packed blocks.  CPU only."""
import numpy as np

import oracle
import synth


def test_splitmix64_published_sequence():
    # splitmix64 seeded with 0: the published first outputs
    assert synth.u64(0, 0) == 0xE220A8397B1DCDAF
    assert synth.u64(0, 1) == 0x6E789E6AA1B965F4
    assert synth.u64(0, 2) == 0x06C45D188009454F


def test_slices_regenerate():
    a = synth.normal(123, (6, 64))
    b = synth.normal(123, (3, 64))
    assert np.array_equal(a[:3], b)
    x = synth.make_acts(synth.CONFIGS[3][3])        # M = 4096 rows
    y = synth.make_acts(synth.CONFIGS[3][0], rows=16)
    assert np.array_equal(x[:16], y)


def test_moments():
    z = synth.normal(9, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    t = synth.student_t4(10, 1 << 20).astype(np.float64)
    assert abs(t.mean()) < 1e-2 and abs(t.var() - 2.0) < 0.2      # var of t_4 is 2
    r = synth.rmsnorm_rows(synth.normal(11, (8, 4096)))
    assert np.allclose(np.sqrt((r.astype(np.float64) ** 2).mean(1)), 1.0, atol=1e-5)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-39], np.float32)
    b = synth.to_bf16_bits(x)
    assert list(b[:3]) == [0x3F80, 0x3F80, 0x3F82]
    assert np.array_equal(synth.bf16_bits_to_f32(b)[3:4], np.float32([-2.5]))


def test_packed_blocks_reconstruct():
    for fmt in (synth.Q4_K, synth.Q6_K):
        w = synth.normal(77, (16, 1024), 0.0, 0.02)
        W = synth.pack(fmt, w)
        wh = oracle.dequant(fmt, W, 16, 1024)
        blocks = np.abs(w.astype(np.float64)).reshape(-1, 32 if fmt == 0 else 16).max(1)
        err = np.abs(wh - w).reshape(blocks.shape[0], -1).max(1)
        assert np.all(err <= 0.15 * blocks + 1e-6), (err / blocks).max()
        assert np.corrcoef(wh.ravel(), w.ravel())[0, 1] > 0.99


def test_random_blocks_have_finite_scales():
    for fmt in (synth.Q4_K, synth.Q6_K):
        W = synth.random_blocks(fmt, 8, 512, seed=3, emin=0, emax=30)
        w = oracle.dequant(fmt, W, 8, 512)
        assert np.all(np.isfinite(w))
