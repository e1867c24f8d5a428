"""The oracle pins have teeth: each plausible mistake, planted in a copy of the oracle
source built on the CPU, makes the pin suite in test_oracle.py fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rehyat_oracle.c")

MUTANTS = {
    "drop_last_power": ("for (int pw = 1; pw <= P; ++pw)", "for (int pw = 1; pw < P + (P == 1); ++pw)"),
    "scale_1_over_D": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "no_overlap": ("ws = f0 - p->To > 0 ? f0 - p->To : 0;", "ws = f0;"),
    "overlap_after": ("we = f1;", "we = f1 + p->To < p->T ? f1 + p->To : p->T;"),
    "no_linear_normaliser": ("double den = a * l + g * z;", "double den = a * l + g;"),
    "relu_not_softplus": ("return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));", "return (x > 0 ? x : 0.0);"),
    "transposed_w": ("acc += w_h[(int64_t)j * D + d] * xt[d];", "acc += w_h[(int64_t)d * Dphi + j] * xt[d];"),
    "z_squared": ("Z[f] += a;", "Z[f] += a * a;"),
    "linear_scale_sign": ("double g = has_lin ? exp(-M) : 0.0;", "double g = has_lin ? exp(M) : 0.0;"),
    "window_includes_next_frame": ("if (f >= ws && f < we) {\n                        s[j]", "if (f >= ws && f <= we) {\n                        s[j]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_pins(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert before in src, f"mutation site for {name} not found"
    msrc = tmp_path / "rehyat_oracle.c"
    msrc.write_text(src.replace(before, after))
    shutil.copy(os.path.join(ROOT, "oracle", "rehyat_oracle.h"), tmp_path / "rehyat_oracle.h")
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(msrc), "-lm"],
                   check=True)
    env = dict(os.environ, REHYAT_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
