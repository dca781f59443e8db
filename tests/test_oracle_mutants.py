"""Plant plausible mistakes into copies of the oracle and check the pins catch each.

Every mutant is a copy of oracle/ternary_oracle.c with one textual change,
built with gcc into a temporary directory (CPU only).  A mutant that passes
every pin would mean the pins do not pin that part of the oracle.
"""

import subprocess
from pathlib import Path

import pytest

import oracle
from oracle_pins import PINS

SRC = Path(oracle.__file__).resolve().parent / "ternary_oracle.c"

MUTANTS = {
    "msb_first_fields": ("return (byte >> (2 * i)) & 3;", "return (byte >> (6 - 2 * i)) & 3;"),
    "swapped_signs": ("CODE_TABLE[4] = {0, 1, -1, 0};", "CODE_TABLE[4] = {0, -1, 1, 0};"),
    "reserved_as_plus": ("CODE_TABLE[4] = {0, 1, -1, 0};", "CODE_TABLE[4] = {0, 1, -1, 1};"),
    "reserved_as_minus": ("CODE_TABLE[4] = {0, 1, -1, 0};", "CODE_TABLE[4] = {0, 1, -1, -1};"),
    "eq_form_wrong": ("return (c == 1) - (c == 2);", "return (c == 1) - (c == 3);"),
    "bits_form_wrong": ("return (c & 1) - ((c >> 1) & 1);", "return (c & 1) + ((c >> 1) & 1) - 2 * (c == 2);"),
    "pack_minus_code": ("code = 2;", "code = 3;"),
    "pack_msb_first": ("(uint8_t)(code << (2 * (k % 4)))", "(uint8_t)(code << (6 - 2 * (k % 4)))"),
    "pack_no_count": ("++invalid;", ";"),
    "row_stride": ("uint8_t byte = packed[n * (K / 4) + k / 4];",
                   "uint8_t byte = packed[n * (K / 8) + k / 4];"),
    "group_index_off_by_one": ("k / group_size]);", "(k + 1) / group_size % (K / group_size)]);"),
    "group_scale_transposed": ("scale[n * (K / group_size) + k / group_size]",
                               "scale[(k / group_size) * (K / group_size) + n % (K / group_size)]"),
    "group_fixed_128": ("scale[n * (K / group_size) + k / group_size]",
                        "scale[n * (K / group_size) + (k / 128) % (K / group_size)]"),
    "per_channel_first_scale": ("return ternary_oracle_f16_to_f64(scale[n]);",
                                "return ternary_oracle_f16_to_f64(scale[0]);"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n                    double xv",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n                    double xv"),
    "sign_of_sum": ("acc += xv * w[k];\n                    b += fabs(xv) * a[k];\n                }\n                y[m * N + n]",
                    "acc -= xv * w[k];\n                    b += fabs(xv) * a[k];\n                }\n                y[m * N + n]"),
    "bound_no_abs": ("b += fabs(xv) * a[k];\n                }\n                y[m * N + n]",
                     "b += xv * a[k];\n                }\n                y[m * N + n]"),
    "x_transposed": ("uint16_t bits = x[m * K + k];", "uint16_t bits = x[k * M + m];"),
    "bf16_bias": ("v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),
    "bf16_no_implicit": ("v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(f), e - 134);"),
    "f16_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "f16_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "sample_wrong_row": ("int64_t m = ms[i], n = ns[i];", "int64_t m = ms[i], n = ns[count - 1 - i];"),
    "census_wrong_code": ("c += field_of(packed[i], f) == 3;", "c += field_of(packed[i], f) == 2;"),
}


def _needs_m(src: str) -> str:
    # x_at() has no M in scope; pass it through for the transposed-x mutant.
    return (src.replace("static double x_at(const uint16_t *x, int x_fp16, int64_t K, int64_t m, int64_t k)",
                        "static int64_t M_glob;\nstatic double x_at(const uint16_t *x, int x_fp16, int64_t K, int64_t m, int64_t k)")
               .replace("x[k * M + m]", "x[k * M_glob + m]")
               .replace("    int used = 1;\n    if (nthreads <= 0)\n        nthreads = 1;\n#pragma omp parallel num_threads(nthreads)\n    {\n#ifdef _OPENMP\n#pragma omp single\n        used = omp_get_num_threads();\n#endif\n        double *w = (double *)malloc(sizeof(double) * (size_t)K);\n        double *a = (double *)malloc(sizeof(double) * (size_t)K);\n#pragma omp for schedule(static)",
                        "    int used = 1;\n    M_glob = M;\n    if (nthreads <= 0)\n        nthreads = 1;\n#pragma omp parallel num_threads(nthreads)\n    {\n#ifdef _OPENMP\n#pragma omp single\n        used = omp_get_num_threads();\n#endif\n        double *w = (double *)malloc(sizeof(double) * (size_t)K);\n        double *a = (double *)malloc(sizeof(double) * (size_t)K);\n#pragma omp for schedule(static)"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = SRC.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new)
    if name == "x_transposed":
        src = _needs_m(src)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, str(c), "-o", str(so), "-lm"])
    mut = oracle.Oracle(so)
    failed = []
    for pin in PINS:
        try:
            pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash-free mutant may still raise, e.g. shape errors
            failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"mutant {name} passes every pin"
