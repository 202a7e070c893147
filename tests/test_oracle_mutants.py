"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin suite against that
build in a child process: the suite has to fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sla_oracle.c")

MUTANTS = {
    "no_softmax_scale": ("acc *= inv_sqrt_d;", ""),
    "pool_divides_by_block": ("out[(bh * Nb + i) * d + c] = (float)(s / (double)n_i);",
                              "out[(bh * Nb + i) * d + c] = (float)(s / (double)blk);"),
    "ties_favour_high_index": ("return (x->j < y->j) ? -1 : (x->j > y->j);",
                               "return (x->j > y->j) ? -1 : (x->j < y->j);"),
    "projection_not_transposed": ("y += ol_t[e] * (double)w[c * d + e];",
                                  "y += ol_t[e] * (double)w[e * d + c];"),
    "linear_not_normalised": ("ol[e] = acc / den;", "ol[e] = acc;"),
    "negligible_from_wrong_end": ("for (long p = Nb - k_n; p < Nb; ++p) mrow[r[p].j] = -1;",
                                  "for (long p = k_c; p < k_c + k_n; ++p) mrow[r[p].j] = -1;"),
    "negligible_leaks_into_linear": ("if (mrow[j] != 0) continue;\n                    ++n_marg;",
                                     "if (mrow[j] == 1) continue;\n                    ++n_marg;"),
    "phi_over_wrong_sign": ("out[c] = exp((double)x[c] - m);", "out[c] = exp(m - (double)x[c]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", str(mut), "-o", str(so), "-lm"])
    env = dict(os.environ, SLA_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
