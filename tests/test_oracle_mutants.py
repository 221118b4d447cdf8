"""The oracle's pins must be strong enough to catch plausible mistakes.

Each case plants one mistake in a private copy of oracle.c (on the CPU, never
in the HIP path), builds it, and runs the pin tests against that build in a
fresh interpreter: at least one pin must fail.  The original oracle passes the
same tests (they are the regular CPU suite).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j] = scale * acc;", "s[j] = acc;", "test_oracle_fwd.py"),
    "lse_sign": ("const double p = exp(s[j] - m);", "const double p = exp(s[j] + m);", "test_oracle_fwd.py"),
    "mask_off_by_one": ("return causal ? i + 1 : N;", "return causal ? i + 2 : N;", "test_oracle_fwd.py"),
    "wrong_operand": ("for (int64_t c = 0; c < d; ++c) acc += q_row[c] * kh[j * d + c];",
                      "for (int64_t c = 0; c < d; ++c) acc += q_row[c] * vh[j * d + c];", "test_oracle_fwd.py"),
    "no_normalise": ("for (int64_t c = 0; c < d; ++c) o_row[c] /= l;", "", "test_oracle_fwd.py"),
    "lse_dropped_max": ("*lse = m + log(l);", "*lse = log(l);", "test_oracle_fwd.py"),
    "bwd_dropped_D": ("const double dsij = pij * (dpij - Dv[flat]);", "const double dsij = pij * dpij;",
                      "test_oracle_bwd.py"),
    "bwd_dk_unscaled": ("odk[c] += scale * dsij * qi[c];", "odk[c] += dsij * qi[c];", "test_oracle_bwd.py"),
    "e4m3_ties_down": ("else pick = (lo % 2 == 0) ? lo : lo + 1;", "else pick = lo;", "test_oracle_fp8.py"),
    "e4m3_bias": ("else mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                  "else mag = ldexp(1.0 + (double)m / 8.0, e - 8);", "test_oracle_fp8.py"),
    "r1_p_unscaled": ("e4m3_decode_one(e4m3_encode_one(p * 256.0)) / 256.0 : p;",
                      "e4m3_decode_one(e4m3_encode_one(p * 256.0)) : p;", "test_oracle_fp8.py"),
    "r1_sum_of_quantised_p": ("l += p;", "l += pw;", "test_oracle_fp8.py"),
    "probs_dropped_scale": ("p_out[j] = scale * acc;", "p_out[j] = acc;", "test_oracle_fwd.py"),
    "probs_wrong_row": ("acc += q[flat_row * d + c] * kh[j * d + c];",
                        "acc += q[(flat_row ^ 1) * d + c] * kh[j * d + c];", "test_oracle_fwd.py"),
    "hadamard_no_signs": ("acc += x[r * d + i] * (double)signs[i] * hadamard_entry(i, j);",
                          "acc += x[r * d + i] * hadamard_entry(i, j);", "test_oracle_fp8.py"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new, suite = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(so), str(mutant_c), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", suite)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
