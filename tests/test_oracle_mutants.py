"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a transposed operand, a
wrong index, a swapped nibble order, a wrong scale index, ties rounded away from
even, a lost ReLU or its sign of zero, wrong special-value handling, and the
same kinds of slip in the E4M3 decode and the MX-format GEMM."""

import os
import shutil

import pytest

import oracle
import oracle_pins

# (name, exact text in oracle.c, replacement, which occurrence (0-based))
MUTANTS = [
    ("gemm_drops_last_k", "yi[j] += a * bk[j];", "yi[j] += a * bk[j] * (k + 1 < K);", 0),
    ("gemm_wrong_sign", "yi[j] += a * bk[j];", "yi[j] -= a * bk[j];", 0),
    ("gemm_transposed_a", "const double a = Ad[i * K + k];", "const double a = Ad[k * M + i];", 0),
    ("dequant_transposed_a", "const double a = Ad[i * K + k];", "const double a = Ad[k * M + i];", 1),
    ("entries_drop_first_k", "s += a * b;", "s += a * b * (k > 0);", 0),
    ("entries_wrong_col_bf16", "b = orc_decode_bf16(((const uint16_t*)B)[k * N + j]);",
     "b = orc_decode_bf16(((const uint16_t*)B)[k * N + (N - 1 - j)]);", 0),
    ("gemm_relu_lost", "yi[j] = relu_f64(yi[j]);", "yi[j] = yi[j];", 0),
    ("relu_negative_zero", "return y > 0.0 ? y : 0.0;", "return y > 0.0 ? y : -0.0;", 0),
    ("dequant_drops_last_k", "yi[j] += a * bk[j];", "yi[j] += a * bk[j] * (k + 1 < K);", 1),
    ("nibble_order_swapped", "(4 * (k % 2))", "(4 * (1 - k % 2))", 1),
    ("scale_index_wrong", "Ws[n * (K / 32) + k / 32]", "Ws[n * (K / 32) + (k / 32 + 1) % (K / 32)]", 0),
    ("ties_away_from_even", "(rem == half && (n & 1ull))", "(rem == half)", 0),
    ("overflow_off_by_one", "if (efield >= emax_field)", "if (efield > emax_field)", 0),
    ("e2m1_has_specials", "decode_bits(code & 0xFu, 2, 1, 0)", "decode_bits(code & 0xFu, 2, 1, 1)", 0),
    ("subnormal_exponent", "v = ldexp((double)f, 1 - bias - fbits);", "v = ldexp((double)f, -bias - fbits);", 0),
    ("e8m0_bias", "ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)", 0),
    ("layout_a_stride", "return trans_a ? Ad[k * M + i] : Ad[i * K + k];",
     "return trans_a ? Ad[i * M + k] : Ad[i * K + k];", 0),
    ("layout_b_stride", "return trans_b ? Bd[j * K + k] : Bd[k * N + j];",
     "return trans_b ? Bd[k * K + j] : Bd[k * N + j];", 0),
    ("layout_entries_a", "const int64_t ia = trans_a ? k * M + i : i * K + k;",
     "const int64_t ia = trans_a ? i * K + k : i * K + k;", 0),
    ("layout_entries_b", "const int64_t ib = trans_b ? j * K + k : k * N + j;",
     "const int64_t ib = trans_b ? k * N + j : k * N + j;", 0),
    ("layout_relu_lost", "Y[i * N + j] = relu ? relu_f64(s) : s;", "Y[i * N + j] = s;", 0),
    ("e4m3_ieee_specials", "return decode_bits(code, 4, 3, 0);", "return decode_bits(code, 4, 3, 1);", 0),
    ("e4m3_positive_nan_only", "if ((code & 0x7Fu) == 0x7Fu)", "if (code == 0x7Fu)", 0),
    ("e4m3_bias_8", "return decode_bits(code, 4, 3, 0);", "return 0.5 * decode_bits(code, 4, 3, 0);", 0),
    ("mx_a_nibble_order", "(4 * (k % 2))", "(4 * (1 - k % 2))", 2),
    ("mx_a_scale_index", "As[m * (K / 32) + k / 32]", "As[m * (K / 32) + (k / 32 + 1) % (K / 32)]", 0),
    ("mx_a_scale_per_16", "As[m * (K / 32) + k / 32]", "As[m * (K / 32) + (k / 16) % (K / 32)]", 0),
    ("mx_e4m3_row_stride", "e = orc_decode_e4m3(Aq[m * K + k]);", "e = orc_decode_e4m3(Aq[m * (K / 2) + k]);", 0),
    ("mx_format_swapped", "if (fmt == 0) {", "if (fmt != 0) {", 0),
    ("mx_gemm_drops_last_k", "yi[j] += a * bk[j];", "yi[j] += a * bk[j] * (k + 1 < K);", 2),
    ("mx_gemm_weight_transposed", "Bd[k * N + n] = w4_value(Wq, Ws, K, n, k);",
     "Bd[k * N + n] = w4_value(Wq, Ws, K, (n + 1) % N, k);", 1),
    ("mx_entries_reversed_k", "s += mx_a_value(fmt, Aq, As, K, i, k) * w4_value(Wq, Ws, K, j, k);",
     "s += mx_a_value(fmt, Aq, As, K, i, k) * w4_value(Wq, Ws, K, j, K - 1 - k);", 0),
    ("mx_relu_lost", "yi[j] = relu_f64(yi[j]);", "yi[j] = yi[j];", 2),
    ("sp24_nibble_order", "(Ai[m * (K / 8) + j / 2] >> (4 * (j % 2)))",
     "(Ai[m * (K / 8) + j / 2] >> (4 * (1 - j % 2)))", 0),
    ("sp24_positions_swapped", "return t == 0 ? (nib & 3) : (nib >> 2);",
     "return t == 0 ? (nib >> 2) : (nib & 3);", 0),
    ("sp24_group_stride", "A[m * K + 4 * j + sp24_pos(Ai, K, m, j, t)] +=",
     "A[m * K + 2 * j + sp24_pos(Ai, K, m, j, t)] +=", 0),
    ("sp24_repeated_overwrites", "A[m * K + 4 * j + sp24_pos(Ai, K, m, j, t)] +=",
     "A[m * K + 4 * j + sp24_pos(Ai, K, m, j, t)] =", 0),
    ("sp24_value_index", "decode_one(dtype, Ac, m * (K / 2) + 2 * j + t);",
     "decode_one(dtype, Ac, m * (K / 2) + 2 * j + (1 - t));", 0),
    ("sp24_entries_k", "const int64_t k = 4 * j + sp24_pos(Ai, K, i, j, t);",
     "const int64_t k = 4 * j + t;", 0),
    ("sp24_relu_lost", "yi[j] = relu_f64(yi[j]);", "yi[j] = yi[j];", 3),
]


def _mutate(text, old, new, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, "mutation target not found: %r" % old
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, occ):
    src = open(oracle.SRC).read()
    bad = _mutate(src, old, new, occ)
    assert bad != src
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(bad)
    lib = oracle.build(force=True, src=str(csrc), out=str(tmp_path / "liboracle_mutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "no pin caught mutant %s" % name
