"""Plant plausible mistakes in copies of the Phase A oracle (on the CPU) and check that its pin battery catches each.

Each mutant is the oracle's C source with one textual change, compiled to a temporary library. A mutant that no pin
fails would mean the pins cannot tell that mistake from the definition.
"""

import os

import pytest

import oracle
from tests import pa2_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gx_pa2_oracle.c")

MUTANTS = {
    "no_acc_reset_at_first": [("                    for (int c = 0; c < PA2_SLICE_MAX; ++c) acc[c] = 0.0f;\n", "")],
    "unfused_acc": [("acc[c] = fmaf(sck, x[c], acc[c]);", "{ volatile float pr = sck * x[c]; acc[c] = pr + acc[c]; }")],
    "unfused_lane_chain": [("    s = fmaf(a[1], b[1], s);", "    { volatile float pr = a[1] * b[1]; s = pr + s; }")],
    "sequential_tree": [("        for (int i = 0; i < PA2_LANES; i += 2 * span) v[i] = v[i] + v[i + span];",
                         "        if (span == 1) for (int i = 1; i < PA2_LANES; ++i) v[0] = v[0] + v[i];")],
    "tree_over_used_lanes_only": [("    for (int span = 1; span < PA2_LANES; span *= 2)",
                                   "    for (int span = 1; span < 4; span *= 2)")],
    "ordinal_counts_invalid_firsts": [("                        ++ordinal;\n", ""),
                                      ("                if (pay & PA2_FIRST) {\n                    for",
                                       "                if (pay & PA2_FIRST) {\n                    if (!valid) ++ordinal;\n"
                                       "                    if (valid) ++ordinal;\n                    for")],
    "beta_sign_dropped": [("(-beta[k * C + t]) * dot", "beta[k * C + t] * dot")],
    "out_g_without_cpe": [("out_g[o] = valid ? cpe * g : 0.0f;", "out_g[o] = valid ? g : 0.0f;")],
    "output_index_transposed": [("const int64_t o = k * n + t * W + w;", "const int64_t o = k * n + w * C + t;")],
    "last_store_without_gdw": [("grad[(int64_t)r[1] * hd + col] = fmaf(gdw[c], cpe, acc[c]);",
                                "grad[(int64_t)r[1] * hd + col] = acc[c];")],
    "bank_gets_gdw": [("bank[(int64_t)r[1] * hd + col] = sn[c];", "bank[(int64_t)r[1] * hd + col] = gdw[c];")],
    "invalid_records_output": [("out_eff[o] = valid ? (-beta[k * C + t]) * dot : 0.0f;",
                                "out_eff[o] = (-beta[k * C + t]) * dot;")],
    "invalid_last_stores": [("if ((pay & PA2_LAST) && valid) {", "if (pay & PA2_LAST) {")],
    "invalid_first_reads_rows": [("                    if (valid) {\n                        const int64_t srow",
                                  "                    if (1) {\n                        const int64_t srow")],
    "slice_width_128": [("const int64_t slw = 4 * (((hd + 3) / 4 + nsl - 1) / nsl);", "const int64_t slw = 128;")],
    "per_entry_row_without_chunk": [
        ("const int64_t srow = ssr < 0 ? k * n + ordinal : ti * ssr + p * C * W + t * W + w;\n                        ++ordinal;",
         "const int64_t srow = ssr < 0 ? k * n + ordinal : ti * ssr + t * W + w;\n                        ++ordinal;")],
    "x_from_token_zero": [("du[(k * C + t) * ld_u + col]", "du[(k * C) * ld_u + col]")],
    "raw_planes_scaled": [("out_eff[sl * plane + o] = valid ? dot : 0.0f;",
                           "out_eff[sl * plane + o] = valid ? (-beta[k * C + t]) * dot : 0.0f;")],
    "guard_never_refuses": [("    if (!fpenv_ok()) return PA2_BAD_FPENV;\n", "")],
    "records_unchecked": [("            if (t >= C || w >= W) return PA2_BAD_RECORD;\n", "")],
}


def _build_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutant {name}: pattern not found: {old!r}"
        src = src.replace(old, new, 1)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    out = str(tmp_path / f"lib_{name}.so")
    oracle.build(str(path), out)
    return oracle.load_pa2(out)


def test_unmutated_oracle_passes_every_pin():
    res = pa2_pins.run_all(oracle.load_pa2())
    assert all(v is None for v in res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    lib = _build_mutant(name, tmp_path)
    res = pa2_pins.run_all(lib)
    caught = [k for k, v in res.items() if v is not None]
    assert caught, f"no pin catches the planted mistake {name!r}"
