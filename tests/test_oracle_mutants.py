"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pin battery catches each one.

Each mutant is the oracle's C source with one textual change, compiled to a temporary library. A mutant that no pin
fails would mean the pins cannot tell that mistake from the definition.
"""

import os

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gx_gemm_oracle.c")

MUTANTS = {
    # name: list of (old, new) replacements
    "transposed_x": [("x[(n * C + j) * C + i]", "x[(n * C + i) * C + j]")],
    "reversed_chain": [("for (int64_t j = 0; j < C; ++j) {", "for (int64_t j = C - 1; j >= 0; --j) {")],
    "short_chain": [("for (int64_t j = 0; j < C; ++j) {", "for (int64_t j = 0; j + 1 < C; ++j) {")],
    "unfused_multiply_add": [("acc = fmaf(xv, dv, acc);", "{ volatile float pr = xv * dv; acc = pr + acc; }")],
    "double_accumulator": [("float acc = +0.0f;", "double acc = +0.0;"),
                           ("acc = fmaf(xv, dv, acc);", "acc = fma((double)xv, (double)dv, acc);")],
    "negative_zero_start": [("float acc = +0.0f;", "float acc = -0.0f;")],
    "chain_starts_at_d_u": [("float acc = +0.0f;", "float acc = d_u[(n * C + i) * ld_u + c];"),
                            ("*u = *u + acc;", "*u = acc;")],
    "dropped_final_add": [("*u = *u + acc;", "*u = acc;")],
    "subtracted_update": [("*u = *u + acc;", "*u = *u - acc;")],
    "flush_subnormals": [("acc = fmaf(xv, dv, acc);",
                          "acc = fmaf(xv, dv, acc); if (fabsf(acc) < 1.17549435e-38f) acc = copysignf(0.0f, acc);")],
    "wrong_step_index": [("const int64_t n = ti * P + p;", "const int64_t n = ti + p;")],
    "ignores_row_stride": [("d_dv[(n * C + j) * ld_dv + c]", "d_dv[(n * C + j) * hd + c]")],
    "writes_padding": [("for (int64_t c = 0; c < hd; ++c) {", "for (int64_t c = 0; c < ld_u; ++c) {")],
    "guard_never_refuses": [("    if (!sdm_gx_oracle_fpenv_ok()) return ORACLE_BAD_FPENV;\n", "")],
    "guard_ignores_flush_to_zero": [("    if (csr & (1u << 15)) return 0;\n", "")],
    "guard_ignores_denormals_are_zero": [("    if (csr & (1u << 6)) return 0;\n", "")],
    "guard_ignores_sse_rounding": [("    if (csr & (3u << 13)) return 0;\n", "")],
    "guard_ignores_c_rounding": [("    if (fegetround() != FE_TONEAREST) return 0;\n", "")],
    "first_product_start": [("float acc = +0.0f;\n                for (int64_t j = 0; j < C; ++j) {",
                             "float acc = x[(n * C) * C + i] * d_dv[(n * C) * ld_dv + c];\n"
                             "                for (int64_t j = 1; j < C; ++j) {")],
}


def _build_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutant {name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    out = str(tmp_path / f"lib_{name}.so")
    oracle.build(str(path), out)
    return oracle.load(out)


def test_unmutated_oracle_passes_every_pin(oracle_lib):
    res = pins.run_all(oracle_lib)
    assert all(v is None for v in res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    lib = _build_mutant(name, tmp_path)
    res = pins.run_all(lib)
    caught = [k for k, v in res.items() if v is not None]
    assert caught, f"no pin catches the planted mistake {name!r}"
