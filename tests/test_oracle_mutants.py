"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mutants are built from the oracle's C source with one textual change
each, compiled to a temporary library, and the pin checks are run against
them (CPU only).  A mutant that passes every pin means the pins have a hole.
"""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qknorm_oracle.c")

MUTANTS = {
    "drop_eps": ("double inv = 1.0 / sqrt(S / n + eps);", "double inv = 1.0 / sqrt(S / n);"),
    "eps_outside_sqrt": ("double inv = 1.0 / sqrt(S / n + eps);",
                         "double inv = 1.0 / (sqrt(S / n) + eps);"),
    "divide_by_shard_width": ("apply_group(x, dtype, row, wq, S, (double)wq,",
                              "apply_group(x, dtype, row, wq, S, (double)(wq / nshards),"),
    "gamma_not_indexed": ("load_value(g, gamma_dtype(dtype), goff + j)", "load_value(g, gamma_dtype(dtype), goff)"),
    "k_heads_use_gamma_q": ("apply_group(x, dtype, off, D, S, (double)D, gamma_k, 0, eps, y, yr);",
                            "apply_group(x, dtype, off, D, S, (double)D, gamma_q, 0, eps, y, yr);"),
    "k_heads_wrong_offset": ("int64_t off = row + wq + (int64_t)h * D;",
                             "int64_t off = row + (int64_t)h * D;"),
    "last_shard_dropped": ("for (int r = 0; r < nshards; ++r)\n        S += sum_of_squares",
                           "for (int r = 0; r + 1 < nshards; ++r)\n        S += sum_of_squares"),
    "apply_drops_a_part": ("for (int r = 0; r < nparts; ++r)\n                S += part_q",
                           "for (int r = 1; r < nparts; ++r)\n                S += part_q"),
    "abs_square_sign": ("s += v * v;", "s += v * fabs(v);"),
    "rounding_truncates": ("double q = nearbyint(ldexp(v, 8 - e));", "double q = trunc(ldexp(v, 8 - e));"),
    "padding_not_copied": ("pass_through(x, dtype, row + wq + wk, ld - wq - wk, y, yr);\n    }\n    return 0;\n}\n\n/* Layerwise",
                           "pass_through(x, dtype, row + wq + wk, ld - wq - wk - 1, y, yr);\n    }\n    return 0;\n}\n\n/* Layerwise"),
    "partials_transposed": ("part_q[(int64_t)r * T + t] = sum_of_squares",
                            "part_q[t * nshards + r] = sum_of_squares"),
    "f16_exponent_bias_off_by_one": ("v = ldexp((double)(1024 + m), e - 25);",
                                     "v = ldexp((double)(1024 + m), e - 24);"),
    "f16_subnormals_flushed": ("v = ldexp((double)m, -24);", "v = 0.0 * m;"),
    "f16_rounding_truncates": ("double q = nearbyint(ldexp(a, 11 - e));",
                               "double q = trunc(ldexp(a, 11 - e));"),
    "f16_overflow_saturates": ("if (r > 65504.0)\n        return sign | 0x7C00;",
                               "if (r > 65504.0)\n        return sign | 0x7BFF;"),
    "f16_stored_as_bf16": ("else if (dtype == 2)\n        ((uint16_t *)p)[i] = round_to_f16(v);",
                           "else if (dtype == 2)\n        ((uint16_t *)p)[i] = round_to_bf16(v);"),
    "e4m3_exponent_bias_off_by_one": ("v = ldexp((double)(8 + m), e - 10);",
                                      "v = ldexp((double)(8 + m), e - 9);"),
    "e4m3_rounding_truncates": ("double q = nearbyint(ldexp(a, 4 - e));",
                                "double q = trunc(ldexp(a, 4 - e));"),
    "e4m3_overflow_to_nan": ("if (a > 448.0)\n        return sign | 0x7E;",
                             "if (a > 448.0)\n        return sign | 0x7F;"),
    "e4m3_gamma_read_as_fp8": ("static int gamma_dtype(int dtype) { return dtype == 3 ? 1 : dtype; }",
                               "static int gamma_dtype(int dtype) { return dtype; }"),
    "gamma_after_divide_by_rms_squared": ("double v = load_value(x, dtype, off + j) * load_value(g, gamma_dtype(dtype), goff + j) * inv;",
                                          "double v = load_value(x, dtype, off + j) * load_value(g, gamma_dtype(dtype), goff + j) * inv * inv;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    cfile = tmp_path / "mutant.c"
    cfile.write_text(mutated)
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(cfile), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_LIB", str(lib))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
