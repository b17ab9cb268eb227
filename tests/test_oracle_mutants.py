"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require every one of them to
fail at least one pin: evidence that the pins constrain each step of the oracle."""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

with open(oracle_build.SOURCE) as _f:
    SOURCE = _f.read()

REDUCE_LOOP = ("    float acc = bf16_to_float(inputs[0][i]);\n"
               "    for (int k = 1; k < n; ++k)\n"
               "        acc = acc + bf16_to_float(inputs[k][i]);\n")

# (name, text in fused_ar_oracle.c, replacement)
MUTANTS = [
    ("reduce_reverse_order", REDUCE_LOOP,
     "    float acc = bf16_to_float(inputs[n - 1][i]);\n"
     "    for (int k = n - 2; k >= 0; --k)\n"
     "        acc = acc + bf16_to_float(inputs[k][i]);\n"),
    ("reduce_pairwise_tree", REDUCE_LOOP,
     "    float part[8];\n"
     "    for (int k = 0; k < n; ++k) part[k] = bf16_to_float(inputs[k][i]);\n"
     "    int cnt = n;\n"
     "    while (cnt > 1) { int h = (cnt + 1) / 2;\n"
     "        for (int k = 0; k + h < cnt; ++k) part[k] = part[k] + part[k + h];\n"
     "        cnt = h; }\n"
     "    float acc = part[0];\n"),
    ("reduce_starts_from_plus_zero", REDUCE_LOOP,
     "    float acc = 0.0f;\n"
     "    for (int k = 0; k < n; ++k)\n"
     "        acc = acc + bf16_to_float(inputs[k][i]);\n"),
    ("reduce_in_binary64", "    float acc = bf16_to_float(inputs[0][i]);\n",
     "    double acc = bf16_to_float(inputs[0][i]);\n"),
    ("reduce_drops_last_rank", "    for (int k = 1; k < n; ++k)\n        acc = acc +",
     "    for (int k = 1; k < n - 1; ++k)\n        acc = acc +"),
    ("round_truncates", "    if (frac > 0.5 || (frac == 0.5 && fmod(lower, 2.0) == 1.0))\n",
     "    if (0)\n"),
    ("round_half_away", "    if (frac > 0.5 || (frac == 0.5 && fmod(lower, 2.0) == 1.0))\n",
     "    if (frac >= 0.5)\n"),
    ("round_ties_to_odd", "fmod(lower, 2.0) == 1.0", "fmod(lower, 2.0) == 0.0"),
    ("round_flushes_subnormals", "    if (q < -133)\n        q = -133;",
     "    if (e < -125)\n        return sign;"),
    ("round_saturates", "    if (r >= 0x1p128)\n        return (uint16_t)(sign | 0x7F80u);",
     "    if (r >= 0x1p128)\n        return (uint16_t)(sign | 0x7F7Fu);"),
    ("round_drops_sign", "    return (uint16_t)(sign | (bits >> 16));",
     "    return (uint16_t)(bits >> 16);"),
    ("residual_added_before_rounding",
     "            uint16_t red = reduce_element(inputs, n, i);\n"
     "            double sum = (double)bf16_to_float(red) + (double)bf16_to_float(residual[i]);\n",
     "            float acc = bf16_to_float(inputs[0][i]);\n"
     "            for (int k = 1; k < n; ++k) acc = acc + bf16_to_float(inputs[k][i]);\n"
     "            double sum = (double)acc + (double)bf16_to_float(residual[i]);\n"),
    ("residual_dropped", " + (double)bf16_to_float(residual[i]);", " + 0.0;"),
    ("residual_subtracted", " + (double)bf16_to_float(residual[i]);",
     " - (double)bf16_to_float(residual[i]);"),
    ("residual_wrong_row", "bf16_to_float(residual[i])", "bf16_to_float(residual[(size_t)j])"),
    ("eps_outside_root", "1.0 / sqrt(mean + (double)eps)", "1.0 / sqrt(mean) + (double)eps"),
    ("eps_dropped", "1.0 / sqrt(mean + (double)eps)", "1.0 / sqrt(mean)"),
    ("eps_squared", "1.0 / sqrt(mean + (double)eps)", "1.0 / sqrt(mean + (double)eps * eps)"),
    ("divisor_hidden_minus_one", "sumsq / (double)hidden", "sumsq / (double)(hidden - 1)"),
    ("sum_not_mean", "sumsq / (double)hidden", "sumsq"),
    ("abs_not_square", "sumsq = sumsq + x * x;", "sumsq = sumsq + fabs(x);"),
    ("square_sum_skips_last", "        for (int j = 0; j < hidden; ++j) {\n            double x = (double)bf16_to_float(residual_out[row + (size_t)j]);\n            sumsq",
     "        for (int j = 0; j < hidden - 1; ++j) {\n            double x = (double)bf16_to_float(residual_out[row + (size_t)j]);\n            sumsq"),
    ("no_root", "1.0 / sqrt(mean + (double)eps)", "1.0 / (mean + (double)eps)"),
    ("weight_one_plus", "double w = (double)bf16_to_float(weight[j]);",
     "double w = 1.0 + (double)bf16_to_float(weight[j]);"),
    ("weight_first_only", "bf16_to_float(weight[j])", "bf16_to_float(weight[0])"),
    ("weight_dropped", "oracle_bf16_round(x * rstd * w)", "oracle_bf16_round(x * rstd)"),
    ("out_sign_lost", "oracle_bf16_round(x * rstd * w)", "oracle_bf16_round(fabs(x * rstd * w))"),
    ("out_times_std", "oracle_bf16_round(x * rstd * w)", "oracle_bf16_round(x / rstd * w)"),
    ("round_nan_to_inf", "        return (uint16_t)(sign | 0x7FC0u);",
     "        return (uint16_t)(sign | 0x7F80u);"),
    ("square_sum_skips_non_finite", "sumsq = sumsq + x * x;",
     "if (isfinite(x)) sumsq = sumsq + x * x;"),
    ("row_stride_off_by_one", "size_t row = (size_t)r * (size_t)hidden;",
     "size_t row = (size_t)r * (size_t)(hidden - 1);"),
]


def test_mutant_texts_are_present():
    for name, old, _ in MUTANTS:
        assert SOURCE.count(old) >= 1, f"mutant {name}: text not found in the oracle source"


def test_unmutated_oracle_passes_every_pin():
    assert oracle_pins.failures(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = tmp_path / f"{name}.c"
    src.write_text(SOURCE.replace(old, new))
    lib = oracle_build.build(source=str(src), output=str(tmp_path / f"lib{name}.so"),
                             extra_flags=["-Wno-error"])
    assert os.path.exists(lib)
    failed = oracle_pins.failures(oracle.Oracle(lib))
    assert failed, f"planted mistake {name} passes every pin"
