"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of the oracle's C source (a
dropped term, a wrong sign, a transposed index or operand, a missing guard),
builds it, and runs the pin suites against that build in a child process.
The pins must fail for every mutant; the clean build must pass.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ncc_oracle.c")
PINS = ["tests/test_oracle_sat.py", "tests/test_oracle_correlate.py"]

MUTANTS = {
    "box_drops_top_left": ("           - tbl_at(S, W, x0 - 1, y1 - 1) + tbl_at(S, W, x0 - 1, y0 - 1);",
                           "           - tbl_at(S, W, x0 - 1, y1 - 1);"),
    "box_wrong_sign": ("           - tbl_at(S, W, x0 - 1, y1 - 1) + tbl_at(S, W, x0 - 1, y0 - 1);",
                       "           + tbl_at(S, W, x0 - 1, y1 - 1) - tbl_at(S, W, x0 - 1, y0 - 1);"),
    "box_transposed_corner": ("- tbl_at(S, W, x1 - 1, y0 - 1)", "- tbl_at(S, W, y0 - 1, x1 - 1)"),
    "box_corner_shifted": ("+ tbl_at(S, W, x0 - 1, y0 - 1);", "+ tbl_at(S, W, x0, y0 - 1);"),
    "table_mixes_tables": ("Q[(size_t)y * W + x] = v * v + tbl_at(Q, W, x - 1, y) + tbl_at(Q, W, x, y - 1)",
                           "Q[(size_t)y * W + x] = v * v + tbl_at(Q, W, x - 1, y) + tbl_at(S, W, x, y - 1)"),
    "table_drops_square": ("Q[(size_t)y * W + x] = v * v +", "Q[(size_t)y * W + x] = v +"),
    "table_exclusive": ("S[(size_t)y * W + x] = v + tbl_at(S, W, x - 1, y)", "S[(size_t)y * W + x] = tbl_at(S, W, x - 1, y)"),
    "table_drops_overlap": ("                                   - tbl_at(S, W, x - 1, y - 1);\n",
                            "                                   ;\n"),
    "numerator_sign": ("int64_t num = K * sumIT - sumI * sumT;", "int64_t num = K * sumIT + sumI * sumT;"),
    "numerator_drops_count": ("int64_t num = K * sumIT - sumI * sumT;", "int64_t num = sumIT - sumI * sumT;"),
    "window_variance_term": ("int64_t varI = K * sumISq - sumI * sumI;", "int64_t varI = K * sumISq - sumI;"),
    "template_variance_term": ("int64_t varT = K * sumTSq - sumT * sumT;", "int64_t varT = K * sumTSq;"),
    "no_zero_variance_guard": ("if (varI == 0 || varT == 0) return 0.0f;", ""),
    "float_sqrt": ("double g = (double)num / sqrt((double)varI * (double)varT);",
                   "double g = (float)num / sqrtf((float)varI * (float)varT);"),
    "template_transposed": ("(int64_t)t[(size_t)j * wT + i]", "(int64_t)t[(size_t)i * hT + j]"),
    "window_offset": ("img[(size_t)(y + j) * W + (x + i)]", "img[(size_t)(y + i) * W + (x + j)]"),
    "box_window_short": ("x, y, x + wT, y + hT);\n    int64_t sumISq", "x, y, x + wT - 1, y + hT);\n    int64_t sumISq"),
}


def _build(tmp_path, name, src_text):
    c = tmp_path / (name + ".c")
    c.write_text(src_text)
    so = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           str(c), "-o", str(so), "-lm"])
    return str(so)


def _run_pins(lib):
    env = dict(os.environ, NCC_ORACLE_MUTANT_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


@pytest.mark.slow
def test_clean_build_passes(tmp_path):
    lib = _build(tmp_path, "clean", open(SRC).read())
    assert _run_pins(lib) == 0


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique: " + name
    lib = _build(tmp_path, name, src.replace(old, new))
    assert _run_pins(lib) != 0, "pins did not catch mutant " + name
