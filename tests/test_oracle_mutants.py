"""Plant plausible mistakes in a copy of the oracle's C source, build each
copy, and check that the pins catch every one (CPU only). The planted copies
live in a temporary directory; the oracle itself is never modified."""

import pathlib

import pytest

import oracle
import pins
from oracle import build as oracle_build

SRC = pathlib.Path(oracle.SOURCE).read_text()

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("nibble_order_swapped", "(blk[2 + j] & 15) : (blk[2 + j - 16] >> 4)",
     "(blk[2 + j] >> 4) : (blk[2 + j - 16] & 15)"),
    ("nibbles_interleaved", "(blk[2 + j] & 15) : (blk[2 + j - 16] >> 4)",
     "((j & 1) ? (blk[2 + j / 2] >> 4) : (blk[2 + j / 2] & 15)) : "
     "((j & 1) ? (blk[2 + j / 2] >> 4) : (blk[2 + j / 2] & 15))"),
    ("zero_point_7", "(double)(q - 8)", "(double)(q - 7)"),
    ("zero_point_dropped", "(double)(q - 8)", "(double)(q)"),
    ("q8_unsigned", "(int8_t)blk[2 + j]", "(uint8_t)blk[2 + j]"),
    ("scale_bytes_swapped", "blk[0] | (blk[1] << 8)", "blk[1] | (blk[0] << 8)"),
    ("scale_sign_dropped", "return sign ? -v : v;", "return v;"),
    ("exponent_bias_off", "e - 25)", "e - 24)"),
    ("subnormal_flushed", "v = ldexp((double)f, -24);", "v = 0.0;"),
    ("subnormal_as_normal", "v = ldexp((double)f, -24);", "v = ldexp((double)(1024 + f), -25);"),
    ("abs_dropped", "abs_acc += fabs(t);", "abs_acc += t;"),
    ("x_index_transposed", "xrow[b * 32 + j]", "xrow[j * (nblocks) + b]"),
    ("x_neighbour", "xrow[b * 32 + j]", "xrow[b * 32 + (j ^ 1)]"),
    ("last_block_dropped", "b < nblocks; ++b", "b < nblocks - 1; ++b"),
    ("q8_block_size_18", "const int64_t bs = fmt == 0 ? 18 : 34;", "const int64_t bs = 18;"),
    ("row_stride_wrong", "one_output(fmt, x + m * K, w + n * row_bytes",
     "one_output(fmt, x + m * K, w + n * (row_bytes - 2)"),
    ("output_transposed", "int64_t m = i / N, n = i % N;", "int64_t n = i / M, m = i % M;"),
    ("x_row_ignored", "one_output(fmt, x + m * K,", "one_output(fmt, x,"),
    ("d_applied_twice", "return d * (double)(q - 8);", "return d * d * (double)(q - 8);"),
    ("f32_accumulation", "acc += t;", "acc = (float)(acc + t);"),
    ("gelu_constant_swapped", "sqrt(2.0 / M_PI)", "sqrt(M_PI / 2.0)"),
    ("gelu_constant_rounded", "const double c = sqrt(2.0 / M_PI);", "const double c = 0.8;"),
    ("gelu_constant_rounded_3", "const double c = sqrt(2.0 / M_PI);", "const double c = 0.797;"),
    ("gelu_cubic_off_10pct", "0.044715 * g * g * g", "0.04 * g * g * g"),
    ("gelu_cubic_term", "0.044715 * g * g * g", "0.44715 * g * g * g"),
    ("gelu_half_dropped", "return 0.5 * g * (1.0 +", "return g * (1.0 +"),
    ("gated_uses_up_twice", "full(0, x, w_gate, M, N, K, g, sg);", "full(0, x, w_up, M, N, K, g, sg);"),
    ("gated_product_is_sum", "h[i] = qmm_oracle_gelu_tanh(g[i]) * u[i];",
     "h[i] = qmm_oracle_gelu_tanh(g[i]) + u[i];"),
    ("gated_activation_on_up", "h[i] = qmm_oracle_gelu_tanh(g[i]) * u[i];",
     "h[i] = g[i] * qmm_oracle_gelu_tanh(u[i]);"),
    ("q4k_scale_min_swapped", "sc[j] = b[j] & 63;\n        mn[j] = b[4 + j] & 63;",
     "sc[j] = b[4 + j] & 63;\n        mn[j] = b[j] & 63;"),
    ("q4k_scale_high_bits_byte", "((b[j - 4] >> 6) << 4)", "((b[j] >> 6) << 4)"),
    ("q4k_min_high_bits_byte", "mn[j] = (b[4 + j] >> 4) | ((b[j] >> 6) << 4);",
     "mn[j] = (b[4 + j] >> 4) | ((b[j - 4] >> 6) << 4);"),
    ("q4k_scale_low_nibble_high", "sc[j] = (b[4 + j] & 15)", "sc[j] = (b[4 + j] >> 4)"),
    ("q4k_nibble_halves_swapped", "(byte & 15) : (byte >> 4)", "(byte >> 4) : (byte & 15)"),
    ("q4k_subblock_index", "const int j = 2 * c + (i >= 32);", "const int j = c + 4 * (i >= 32);"),
    ("q4k_min_added", "- dmin * (double)mn[j]", "+ dmin * (double)mn[j]"),
    ("q4k_dmin_is_d", "(uint16_t)(blk[2] | (blk[3] << 8))", "(uint16_t)(blk[0] | (blk[1] << 8))"),
    ("q4k_nibble_byte_stride", "blk[16 + 32 * c + (i % 32)]", "blk[16 + 16 * c + (i % 32)]"),
    ("q4k_superblock_144_as_128", "const uint8_t *blk = wrow + b * 144;",
     "const uint8_t *blk = wrow + b * 128;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new, 1))
    lib = oracle_build.build(src, tmp_path / "libmutant.so", werror=False)
    failed = pins.failures(oracle.Oracle(lib), quick=True)
    assert failed, f"no pin catches mutant {name}"
