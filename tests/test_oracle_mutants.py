"""Plant plausible mistakes in copies of the oracle; the pins must catch each.

Each mutant is a text substitution, at the first matching site, in
``oracle/rmsnorm_oracle.c`` compiled into a temporary library on the CPU.  A pin set that lets a mutant through would
not have caught that mistake in the real oracle either.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "divisor_padded_width": [("ss / (double)N", "ss / (double)(N + 1)")],
    "divisor_rows": [("ss / (double)N", "ss / (double)(M > 0 ? M : 1)")],
    "eps_dropped": [("sqrt(ms + e)", "sqrt(ms)")],
    "eps_outside_root": [("1.0 / sqrt(ms + e)", "1.0 / (sqrt(ms) + e)")],
    "eps_added_to_sum": [("ss / (double)N", "(ss + e) / (double)N"), ("sqrt(ms + e)", "sqrt(ms)")],
    "sqrt_not_reciprocal": [("const double r = 1.0 / sqrt(ms + e);", "const double r = sqrt(ms + e);")],
    "rstd_stored_as_root": [("rstd[m] = r;", "rstd[m] = 1.0 / r;")],
    "sum_of_abs": [("ss += xv * xv;", "ss += fabs(xv);")],
    "fp32_accumulation": [("double ss = 0.0;", "float ss = 0.0f;")],
    "offset_ignored": [("(off + oracle_decode(w[j], dtype))", "(oracle_decode(w[j], dtype))")],
    "offset_rounded_to_dtype": [("const double off = (double)offset;",
                                 "const double off = oracle_decode(oracle_encode_rne((double)offset, dtype), dtype);")],
    "weight_reversed": [("xv * r * (off + oracle_decode(w[j], dtype))", "xv * r * (off + oracle_decode(w[N - 1 - j], dtype))")],
    "weight_indexed_by_row": [("xv * r * (off + oracle_decode(w[j], dtype))", "xv * r * (off + oracle_decode(w[m % N], dtype))")],
    "x_transposed": [("xr[j]", "x[j * M + m]")],
    "ties_away_from_zero": [("(r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))", "(r >= 0.5)")],
    "truncation": [("(r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))", "(0)")],
    "double_rounding_via_fp32": [("oracle_encode_rne(ye, dtype)", "oracle_encode_rne((double)(float)ye, dtype)")],
    "decode_bias_off_by_one": [("const int bias = (1 << (f.exp_bits - 1)) - 1;\n    const unsigned sign",
                                "const int bias = (1 << (f.exp_bits - 1));\n    const unsigned sign")],
    "decode_flushes_subnormals": [("mag = ldexp((double)frac, 1 - bias - f.frac_bits);", "mag = 0.0;")],
    "encode_flushes_subnormals": [("if (ex < emin) ex = emin;", "if (ex < emin) return (uint16_t)sign;")],
    "encode_saturates_overflow": [("        bits = inf_bits;\n", "        bits = inf_bits - 1;\n")],
    "encode_drops_sign": [("const uint32_t sign = signbit(v) ? 0x8000u : 0u;", "const uint32_t sign = 0u;")],
    # backward
    "bwd_second_term_sign": [("const double v = r * (gk * dyk - r * r * c * xk);",
                              "const double v = r * (gk * dyk + r * r * c * xk);")],
    "bwd_r_not_cubed": [("const double v = r * (gk * dyk - r * r * c * xk);",
                         "const double v = r * (gk * dyk - c * xk);")],
    "bwd_c_without_weight": [("const double t = oracle_decode(dyr[j], dtype) * (off + oracle_decode(w[j], dtype)) *",
                              "const double t = oracle_decode(dyr[j], dtype) * 1.0 *")],
    "bwd_first_term_without_weight": [("const double v = r * (gk * dyk - r * r * c * xk);",
                                       "const double v = r * (dyk - r * r * c * xk);")],
    "bwd_divisor_padded": [("c /= (double)N;", "c /= (double)(N + 1);")],
    "bwd_offset_ignored": [("const double gk = off + oracle_decode(w[k], dtype);",
                            "const double gk = oracle_decode(w[k], dtype);")],
    "bwd_dw_without_rstd": [("oracle_decode(x[m * N + j], dtype) *\n                                 rstd[m];",
                             "oracle_decode(x[m * N + j], dtype) *\n                                 1.0;")],
    "bwd_dw_times_weight": [("oracle_decode(x[m * N + j], dtype) *\n                                 rstd[m];",
                             "oracle_decode(x[m * N + j], dtype) *\n                                 rstd[m] * (off + oracle_decode(w[j], dtype));")],
    "bwd_dw_wrong_row_stride": [("oracle_decode(dy[m * N + j], dtype)", "oracle_decode(dy[m + j * M], dtype)")],
    # backward on fp64 inputs (the fp32 path)
    "bwd_f64_second_term_sign": [("const double v = r * (gk * dyr[k] - r * r * c * xr[k]);",
                                  "const double v = r * (gk * dyr[k] + r * r * c * xr[k]);")],
    "bwd_f64_c_without_weight": [("const double t = dyr[j] * (offset + w[j]) * xr[j];",
                                  "const double t = dyr[j] * xr[j];")],
    "bwd_f64_offset_ignored": [("const double gk = offset + w[k];", "const double gk = w[k];")],
    "bwd_f64_dw_without_rstd": [("const double t = dy[m * N + j] * x[m * N + j] * rstd[m];",
                                 "const double t = dy[m * N + j] * x[m * N + j];")],
    "bwd_f64_divisor_rows": [("c /= (double)N;\n        cabs /= (double)N;\n        for (int64_t k = 0; k < N; ++k) {\n            const double gk = offset",
                              "c /= (double)M;\n        cabs /= (double)N;\n        for (int64_t k = 0; k < N; ++k) {\n            const double gk = offset")],
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    text = source
    for old, new in MUTANTS[name]:
        assert text.count(old) >= 1, f"mutation site for {name} not found: {old!r}"
        text = text.replace(old, new, 1)     # the first site: the forward precedes the backward
    assert text != source, f"mutant {name} changes nothing"
    src = os.path.join(tmp_path, f"mutant_{name}.c")
    with open(src, "w") as f:
        f.write(text)
    lib = oracle.compile_oracle(src, os.path.join(tmp_path, f"libmutant_{name}.so"))
    o = oracle.Oracle(lib)
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            return
    pytest.fail(f"mutant {name} passed every pin")
