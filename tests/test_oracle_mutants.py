"""Mutation check of the oracle's pins (CPU).

Each case plants one plausible mistake in a copy of oracle/ssm_oracle.c (a
dropped term, a wrong sign, index or operand, a misplaced bias, an ignored
input), builds the copy, and runs the pins of tests/test_oracle_pins.py
against it: every mutant must make at least one pin fail.  An unaltered copy
built the same way must pass them all, so a failure is the mutant's doing.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in ssm_oracle.c, replacement); each text occurs exactly once
MUTANTS = [
    ("bias_outside_softplus",
     "double x = delta[i] + (delta_bias ? delta_bias[d] : 0.0);\n"
     "                const double dt = delta_softplus ? sp(x) : x;",
     "double x = delta[i];\n"
     "                const double dt = (delta_softplus ? sp(x) : x) + (delta_bias ? delta_bias[d] : 0.0);"),
    ("s6_no_skip", "if (Dskip) acc += Dskip[d] * ut;", ";"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("A_transposed", "const double a = A[d * N + n];", "const double a = A[n * D + d];"),
    ("s6_ignores_h0", "h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("zoh_inverted", "if (zoh && a != 0.0)", "if (!zoh && a != 0.0)"),
    ("s6_readout_uses_B", "acc += Cm[r + n] * h[n];", "acc += Bm[r + n] * h[n];"),
    ("s6_decay_without_delta", "const double dA = exp(dt * a);", "const double dA = exp(a);"),
    ("s6_input_one_token_late", "const double ut = u[i];",
     "const double ut = t > 0 ? u[i - D] : 0.0;"),
    ("ssd_wrong_group", "g = hh / heads_per_group;", "g = hh % G;"),
    ("ssd_input_without_delta", "const double w = dt * xt[p];", "const double w = xt[p];"),
    ("ssd_decay_without_delta", "const double a = exp(dt * A[hh]);", "const double a = exp(A[hh]);"),
    ("ssd_readout_before_update",
     "row[n] = a * row[n] + w * bt[n];\n                        acc += ct[n] * row[n];",
     "acc += ct[n] * row[n];\n                        row[n] = a * row[n] + w * bt[n];"),
    ("ssd_skip_wrong_index", "if (Dskip) acc += Dskip[hh] * xt[p];",
     "if (Dskip) acc += Dskip[hh] * xt[0];"),
    ("ssd_ignores_h0", "S[k] = h0 ? h0[(b * H + hh) * P * N + k] : 0.0;", "S[k] = 0.0;"),
]


def _build(src_text: str, path: str) -> None:
    c = path[:-3] + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", path, c,
                    "-lm"], check=True)


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, SSM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p",
                           "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_every_mutant_fails_a_pin(tmp_path):
    src = open(SRC).read()
    libs = {"control": str(tmp_path / "control.so")}
    _build(src, libs["control"])
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"{name}: mutation site not unique in ssm_oracle.c"
        libs[name] = str(tmp_path / f"{name}.so")
        _build(src.replace(old, new), libs[name])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        runs = dict(zip(libs, pool.map(_run_pins, libs.values())))
    ctl = runs.pop("control")
    assert ctl.returncode == 0, "the unaltered oracle fails its pins:\n" + ctl.stdout[-2000:]
    survivors = [name for name, r in runs.items() if r.returncode == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
