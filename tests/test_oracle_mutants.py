"""The pins have teeth: plant plausible mistakes in copies of the oracle (on the CPU), rebuild, and
check that at least one pin fails for each.

The first mutant is the defect the "PN weight format" page records for the CPU dot product in
"Where PN runs": shifting by element index instead of pair index.
"""
import os
import shutil
import tempfile

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "pn_oracle.c")

MUTANTS = {
    # name: (original text, planted text, test modules whose pins must catch it)
    "element_index_shift": ("int shift = bits * (t >> 1) + 16 * (t & 1);",
                            "int shift = bits * t;",
                            ["test_oracle_pn.py"]),
    "distributive_decode": ("out[b * G + e] = d * (float)(codes[e] - z);",
                            "out[b * G + e] = d * (float)codes[e] - d * (float)z;",
                            ["test_oracle_pn.py"]),
    "validation_forgets_bit15": ("if (rd_le32(blk + 2 + 4 * i) & 0x80008000u)",
                                 "if (rd_le32(blk + 2 + 4 * i) & 0x80000000u)",
                                 ["test_oracle_pn.py"]),
    "sigma_flipped": ("double sigma = (fabs(mn) > mx) ? 1.0 : -1.0;",
                      "double sigma = (fabs(mn) > mx) ? -1.0 : 1.0;",
                      ["test_oracle_quantizer.py"]),
    "pn_tie_keeps_the_smaller_m": ("        if (err <= best) {",
                                   "        if (err < best) {",
                                   ["test_oracle_quantizer.py"]),
    "nvfp4_tie_keeps_the_later_multiplier": (
        "if (err < best) {\n                    best = err;\n                    best_s = sw;",
        "if (err <= best) {\n                    best = err;\n                    best_s = sw;",
        ["test_oracle_nvfp4.py"]),
    "multiplier_grid_shifted": ("double m = (50 + 2 * i) / 100.0;",
                                "double m = (52 + 2 * i) / 100.0;",
                                ["test_oracle_quantizer.py"]),
    "rint_truncates": ("double q = rint(w / s) + z;",
                       "double q = trunc(w / s) + z;",
                       ["test_oracle_quantizer.py"]),
    "gemv_drops_zero_point": ("double wv = (double)(d * (float)(codes[e] - z));",
                              "double wv = (double)(d * (float)codes[e]);",
                              ["test_oracle_gemv.py"]),
    "f16_subnormal_flushed": ("v = ldexp((double)m, -24);",
                              "v = 0.0 * m;",
                              ["test_oracle_codecs.py"]),
    "e2m1_grid_wrong": ("double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);",
                        "double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e);",
                        ["test_oracle_codecs.py"]),
    "nvfp4_clip_keeps_last_multiplier_only": ("for (int i = 0; i < 5; i++) {",
                                               "for (int i = 4; i < 5; i++) {",
                                               ["test_oracle_nvfp4.py"]),
    "fp8row_scale_divides": ("            out[n * K + k] = c32 * s32;",
                             "            out[n * K + k] = c32 / s32;",
                             ["test_oracle_fp8row.py"]),
    "fp8row_zero_scale_clause_dropped": ("            if (s == 0 && (c & 0x7F) != 0)\n                ok = 0;",
                                         "",
                                         ["test_oracle_fp8row.py"]),
    "hadamard_sign_from_or": ("acc += (popcount64((uint64_t)(i & j)) & 1) ? -xs[j] : xs[j];",
                              "acc += (popcount64((uint64_t)(i | j)) & 1) ? -xs[j] : xs[j];",
                              ["test_oracle_hadamard.py"]),
    "rotated_gemv_drops_zero_point": ("double w_nk = (double)(d * (float)(codes[e] - z));",
                                      "double w_nk = (double)(d * (float)codes[e]);",
                                      ["test_oracle_hadamard.py"]),
    "hadamard_unnormalised": ("const double inv = 1.0 / sqrt((double)B);",
                              "const double inv = 1.0;",
                              ["test_oracle_hadamard.py"]),
    "hadamard_every_slice_reads_the_first": ("const double *xs = x + m * K + base;",
                                             "const double *xs = x + m * K;",
                                             ["test_oracle_hadamard.py"]),
    "bf16_rounding_truncates": ("    double r = rint(ldexp(a, 7 - E)); /* in [128, 256] */",
                                "    double r = floor(ldexp(a, 7 - E)); /* in [128, 256] */",
                                ["test_oracle_fp8row.py"]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    orig, planted, modules = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not found exactly once"
    tmp = tempfile.mkdtemp(prefix="pn_mutant_")
    try:
        msrc = os.path.join(tmp, "pn_oracle.c")
        with open(msrc, "w") as f:
            f.write(src.replace(orig, planted))
        so = oracle.build(out=os.path.join(tmp, "liboracle_mutant.so"), src=msrc)
        import subprocess
        import sys
        here = os.path.dirname(os.path.abspath(__file__))
        env = dict(os.environ, PN_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            *[os.path.join(here, m) for m in modules]],
                           env=env, capture_output=True, text=True, cwd=os.path.dirname(here))
        assert r.returncode != 0, f"mutant {name} survived:\n{r.stdout[-2000:]}"
        assert "failed" in r.stdout, r.stdout[-2000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
