"""Plant plausible mistakes in a copy of oracle.c and require that the pins catch
each one.  The mutants are built into a temporary directory on the CPU; the real
oracle source is never modified."""
import os
import tempfile

import pytest

import oracle
import pins

# (name, exact text in oracle.c, replacement) -- each a mistake a reader of the
# block layout or of the method could plausibly make
MUTANTS = [
    ("q4k_scale_high_bits_from_wrong_byte",
     "sc[j] = (uint8_t)((s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4));",
     "sc[j] = (uint8_t)((s[j + 4] & 0x0F) | ((s[j] >> 6) << 4));"),
    ("q4k_min_low_bits_wrong_nibble",
     "m[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));",
     "m[j] = (uint8_t)((s[j + 4] & 0x0F) | ((s[j] >> 6) << 4));"),
    ("q4k_nibble_order_swapped",
     "q[v] = (v % 64) < 32 ? (byte & 0x0F) : (byte >> 4);",
     "q[v] = (v % 64) < 32 ? (byte >> 4) : (byte & 0x0F);"),
    ("q4k_byte_index_wrong",
     "uint8_t byte = qs[32 * (v / 64) + (v % 32)];",
     "uint8_t byte = qs[(v / 2) % 128];"),
    ("q4k_min_term_sign",
     "acc += dxb * (d * sc * (double)I - dmin * m * (double)Sx[i * nb32 + b]);",
     "acc += dxb * (d * sc * (double)I + dmin * m * (double)Sx[i * nb32 + b]);"),
    ("q4k_min_term_dropped",
     "acc += dxb * (d * sc * (double)I - dmin * m * (double)Sx[i * nb32 + b]);",
     "acc += dxb * (d * sc * (double)I);"),
    ("q6k_qh_shift",
     "int hi = (qh[32 * half + l] >> (2 * quarter)) & 3;",
     "int hi = (qh[32 * half + l] >> quarter) & 3;"),
    ("q6k_ql_half_stride",
     "uint8_t lowbyte = ql[64 * half + 32 * (quarter % 2) + l];",
     "uint8_t lowbyte = ql[32 * half + 32 * (quarter % 2) + l];"),
    ("q6k_offset_dropped_in_gemm",
     "for (int t = 0; t < 16; t++) Ia += ((int32_t)wq[32 * b + t] - 32) * (int32_t)xq[32 * b + t];",
     "for (int t = 0; t < 16; t++) Ia += ((int32_t)wq[32 * b + t]) * (int32_t)xq[32 * b + t];"),
    ("q6k_second_scale_index",
     "acc += dxb * d * ((double)sc[2 * b] * (double)Ia + (double)sc[2 * b + 1] * (double)Ib);",
     "acc += dxb * d * ((double)sc[2 * b] * (double)Ia + (double)sc[2 * b] * (double)Ib);"),
    ("q6k_scale_unsigned",
     "for (int s = 0; s < 16; s++) sc[s] = (int8_t)blk[192 + s];",
     "for (int s = 0; s < 16; s++) sc[s] = (int8_t)(blk[192 + s] & 0x7F);"),
    ("half_exponent_bias",
     "else v = ldexp((double)(f | 0x400), e - 25);",
     "else v = ldexp((double)(f | 0x400), e - 24);"),
    ("half_subnormal_scale",
     "if (e == 0) v = ldexp((double)f, -24);",
     "if (e == 0) v = ldexp((double)f, -25);"),
    ("quant_divisor_128",
     "float d = amax / 127.0f;",
     "float d = amax / 128.0f;"),
    ("quant_truncates",
     "float r = rintf(v);",
     "float r = truncf(v);"),
    ("quant_rounds_half_away",
     "float r = rintf(v);",
     "float r = roundf(v);"),
    ("quant_sum_of_magnitudes",
     "S += qi;",
     "S += qi < 0 ? -qi : qi;"),
    ("gemm_activation_scale_wrong_block",
     "double dxb = (double)dx[i * nb32 + b];",
     "double dxb = (double)dx[i * nb32 + (b ^ 1)];"),
    ("gemm_superblock_index",
     "double d = dw[j * nsb + b / 8];",
     "double d = dw[j * nsb + b / 16];"),
    ("gemm_activation_reversed_in_block",
     "for (int t = 0; t < 32; t++) I += (int32_t)wq[32 * b + t] * (int32_t)xq[32 * b + t];",
     "for (int t = 0; t < 32; t++) I += (int32_t)wq[32 * b + t] * (int32_t)xq[32 * b + 31 - t];"),
    ("partials_offset_dropped",
     "acc += ((int32_t)qw[n * K + b * L + t] - off) * (int32_t)qx[mi * K + b * L + t];",
     "acc += ((int32_t)qw[n * K + b * L + t]) * (int32_t)qx[mi * K + b * L + t];"),
    ("f16_ties_away_from_zero",
     "r = keep + ((rem > half || (rem == half && (keep & 1))) ? 1 : 0);",
     "r = keep + ((rem >= half) ? 1 : 0);"),
    ("f16_no_subnormal_floor",
     "int qe = ev - 10 < -24 ? -24 : ev - 10;",
     "int qe = ev - 10;"),
    ("f16_exponent_bias",
     "int ebits = qe + 25;",
     "int ebits = qe + 24;"),
    ("deq_f16_min_sign",
     "int64_t D = a * q[32 * j + t] * ((int64_t)1 << (ea - e0)) - b * ((int64_t)1 << (eb - e0));",
     "int64_t D = a * q[32 * j + t] * ((int64_t)1 << (ea - e0)) + b * ((int64_t)1 << (eb - e0));"),
    ("deq_f16_neighbour_scale",
     "f16_split(oracle_f64_to_f16(d * sc[j]), &a, &ea);     /* d*sc is exact in fp64 */",
     "f16_split(oracle_f64_to_f16(d * sc[j ^ 1]), &a, &ea);"),
    ("deq_f16_q6_offset_dropped",
     "o[16 * s + t] = f16_round_scaled(a * ((int64_t)q[16 * s + t] - 32), ea);",
     "o[16 * s + t] = f16_round_scaled(a * ((int64_t)q[16 * s + t]), ea);"),
    ("a256_divisor_128",
     "            float d = amax / 127.0f;\n            float id = 1.0f / d;\n            for (int j = 0; j < 8; j++) {",
     "            float d = amax / 128.0f;\n            float id = 1.0f / d;\n            for (int j = 0; j < 8; j++) {"),
    ("a256_sum_over_superblock",
     "                So[j] = S;\n",
     "                So[j] = S + (j > 0 ? So[j - 1] : 0);\n"),
    ("a256_min_term_dropped",
     "                    part += dw[j * nsb + sb] * (double)scw[j * nb32 + b] * (double)I -\n                            dmw[j * nsb + sb] * (double)mw[j * nb32 + b] * (double)Sx[i * nb32 + b];",
     "                    part += dw[j * nsb + sb] * (double)scw[j * nb32 + b] * (double)I;"),
    ("a256_scale_of_next_superblock",
     "                acc += (double)dx[i * nsb + sb] * part;",
     "                acc += (double)dx[i * nsb + (sb + 1) % nsb] * part;"),
    ("q5k_high_bit_from_wrong_pair",
     "q[v] = (uint8_t)(q[v] | (((qh[v % 32] >> (v / 32)) & 1) << 4));",
     "q[v] = (uint8_t)(q[v] | (((qh[v % 32] >> (v / 64)) & 1) << 4));"),
    ("q5k_high_bit_weight",
     "q[v] = (uint8_t)(q[v] | (((qh[v % 32] >> (v / 32)) & 1) << 4));",
     "q[v] = (uint8_t)(q[v] | (((qh[v % 32] >> (v / 32)) & 1) << 5));"),
    ("q5k_nibbles_read_from_qh",
     "decode_nibbles(blk + 48, q);",
     "decode_nibbles(blk + 16, q);"),
    ("q5k_block_stride",
     "decode_q5k_block(W + i * 176, q + i * 256, sc + i * 8, m + i * 8, d + i, dmin + i);",
     "decode_q5k_block(W + i * 144, q + i * 256, sc + i * 8, m + i * 8, d + i, dmin + i);"),
    ("q80_codes_unsigned",
     "for (int t = 0; t < 32; t++) q[i * 32 + t] = (int8_t)blk[2 + t];",
     "for (int t = 0; t < 32; t++) q[i * 32 + t] = (int8_t)(blk[2 + t] & 0x7F);"),
    ("q80_scale_from_codes",
     "d[i] = oracle_half_to_double(rd16(blk));",
     "d[i] = oracle_half_to_double(rd16(blk + 32));"),
    ("q80_gemm_first_block_scale",
     "acc += dxb * dw[j * nb32 + b] * (double)I;",
     "acc += dxb * dw[j * nb32 + b / 8 * 8] * (double)I;"),
    ("rms_mean_not_divided",
     "double v = ss / (double)K + (double)eps;",
     "double v = ss + (double)eps;"),
    ("rms_eps_dropped",
     "double v = ss / (double)K + (double)eps;",
     "double v = ss / (double)K;"),
    ("rms_no_square_root",
     "return (float)(1.0 / sqrt(v));",
     "return (float)(1.0 / v);"),
    ("rms_band_too_narrow",
     "double delta = 2.0 * (double)(K + 1) * ldexp(1.0, -53);",
     "double delta = 0.0;"),
    ("rms_weight_dropped",
     "xn[i * K + k] = t * g[k];",
     "xn[i * K + k] = t;"),
    ("rms_weight_reversed",
     "xn[i * K + k] = t * g[k];",
     "xn[i * K + k] = t * g[K - 1 - k];"),
    ("rms_squares_of_row_zero",
     "double xv = (double)load_x(x, x_dtype, i * K + k);",
     "double xv = (double)load_x(x, x_dtype, k);"),
    ("swiglu_logistic_sign",
     "double silu = z / (1.0 + exp(-z));",
     "double silu = z / (1.0 + exp(z));"),
    ("swiglu_gate_up_swapped",
     "        double z = gate[i];\n        double silu = z / (1.0 + exp(-z));\n        h[i] = silu * up[i];",
     "        double z = up[i];\n        double silu = z / (1.0 + exp(-z));\n        h[i] = silu * gate[i];"),
    ("gemm_f16_abs_sum_signed",
     "aabs += fabs(p);",
     "aabs += p;"),
]


def _fails_some_pin(orc):
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(oracle.source_path()).read()
    assert src.count(old) >= 1, f"mutation site for {name} no longer in oracle.c"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "oracle_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(src=path, out=os.path.join(d, "liboracle_mutant.so"))
        caught = _fails_some_pin(oracle.Oracle(lib))
    assert caught is not None, f"no pin catches mutant {name}"
