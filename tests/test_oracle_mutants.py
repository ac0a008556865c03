"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows the pins have teeth: a dropped term, a wrong sign, a transposed or
mis-strided operand, SiLU on the wrong branch, a lost precision step or a
wrong rounding mode would not go unnoticed.  Mistakes are planted only in
temporary copies of the oracle's C source, built with gcc, on the CPU.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "exp_sign": ("exp(-z)", "exp(z)"),
    "silu_on_up": ("if (c->h) c->h[o] = oracle_silu(ag[b]) * au[b]", "if (c->h) c->h[o] = oracle_silu(au[b]) * ag[b]"),
    "no_silu": ("if (c->h) c->h[o] = oracle_silu(ag[b]) * au[b]", "if (c->h) c->h[o] = ag[b] * au[b]"),
    "sigmoid_not_silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "down_transposed": ("double w = widen_bf16(rd[n]);",
                        "double w = widen_bf16(c->wd[(size_t)n * M + m]);"),
    "gate_up_drops_last_k": ("for (int k = 0; k < K; ++k) {\n            double wg = widen_bf16(rg[k]);",
                             "for (int k = 0; k < K - 1; ++k) {\n            double wg = widen_bf16(rg[k]);"),
    "down_drops_last_n": ("for (int n = 0; n < N; ++n) {\n            double w = widen_bf16(rd[n]);",
                          "for (int n = 0; n < N - 1; ++n) {\n            double w = widen_bf16(rd[n]);"),
    "x_batch_stride": ("double wu = widen_bf16(ru[k]);\n            for (int b = 0; b < B; ++b) {\n                double xv = c->xd[(size_t)b * K + k];",
                       "double wu = widen_bf16(ru[k]);\n            for (int b = 0; b < B; ++b) {\n                double xv = c->xd[(size_t)b + k];"),
    "h_rounded_fp32": ("c->h[o] = oracle_silu(ag[b]) * au[b];",
                       "c->h[o] = (float)(oracle_silu(ag[b]) * au[b]);"),
    "y_stored_transposed": ("acc[b] += c->h[(size_t)b * N + n] * w;\n        }\n        for (int b = 0; b < B; ++b) c->y[(size_t)b * M + (size_t)m] = acc[b];\n    }\n    free(acc);\n}\n\n/*\n * The separate down",
                            "acc[b] += c->h[(size_t)b * N + n] * w;\n        }\n        for (int b = 0; b < B; ++b) c->y[(size_t)m * B + (size_t)b] = acc[b];\n    }\n    free(acc);\n}\n\n/*\n * The separate down"),
    "bf16_truncates": ("nearbyint(a / q)", "floor(a / q)"),
    "rmsnorm_sum_not_mean": ("double inv = 1.0 / sqrt(ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            xn[",
                             "double inv = 1.0 / sqrt(ss + eps);\n        for (int k = 0; k < d_model; ++k)\n            xn["),
    "rmsnorm_no_eps": ("double inv = 1.0 / sqrt(ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            xn[",
                       "double inv = 1.0 / sqrt(ss / (double)d_model);\n        for (int k = 0; k < d_model; ++k)\n            xn["),
    "rmsnorm_no_sqrt": ("double inv = 1.0 / sqrt(ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            xn[",
                        "double inv = 1.0 / (ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            xn["),
    "rescale_eps_outside_sqrt": ("double inv = 1.0 / sqrt(ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            x_next[",
                                 "double inv = 1.0 / sqrt(ss / (double)d_model) + eps;\n        for (int k = 0; k < d_model; ++k)\n            x_next["),
    "rescale_no_eps": ("double inv = 1.0 / sqrt(ss / (double)d_model + eps);\n        for (int k = 0; k < d_model; ++k)\n            x_next[",
                       "double inv = 1.0 / sqrt(ss / (double)d_model);\n        for (int k = 0; k < d_model; ++k)\n            x_next["),
    "rmsnorm_gain_first_only": ("* widen_bf16(gain[k])", "* widen_bf16(gain[0])"),
    "rmsnorm_batch_stride": ("const uint16_t *row = x + (size_t)b * d_model;", "const uint16_t *row = x + (size_t)b;"),
    "fp8_bias_8": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "fp8_no_subnormals": ("(e == 0) ? ldexp((double)m, -9)", "(e == 0) ? 0.0"),
    "fp8_gate_scale_ignored": ("const double sg = (double)c->sg[n], su", "const double sg = 1.0, su"),
    "fp8_down_scale_by_column": ("double w = s * oracle_e4m3_to_double(rd[n]);",
                                 "double w = (double)c->sd[n % M] * oracle_e4m3_to_double(rd[n]);"),
    "fp8_up_codes_from_gate": ("double wu = su * oracle_e4m3_to_double(ru[k]);",
                               "double wu = su * oracle_e4m3_to_double(rg[k]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / f"libmutant_{name}.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, f"no pin caught the planted mistake {name}"
