"""The pins must reject a wrong oracle: each case plants one plausible
mistake in a copy of oracle/ssm_oracle.c (on the CPU), builds it, and runs the
pin suite against it in a subprocess, which must fail.  A pin suite that let
one of these through would not be pinning the oracle."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTATIONS = {
    "scan_decay_sign": ("                        const double abar = exp(delta * a);",
                        "                        const double abar = exp(-delta * a);"),
    "update_decay_sign": ("                    const double abar = exp(delta * a);\n"
                          "                    const double bx = delta * Bv[n] * xv;",
                          "                    const double abar = exp(-delta * a);\n"
                          "                    const double bx = delta * Bv[n] * xv;"),
    "update_state_not_carried": ("const double hn = abar * state[so + n] + bx;",
                                 "const double hn = abar * 0.0 * state[so + n] + bx;"),
    "bias_dropped": ("const double v = dtr[t] + (dt_bias ? dt_bias[hd] : 0.0);",
                     "const double v = dtr[t];"),
    "taps_reversed": ("weight[(size_t)c * width + k] * XT(t - hist + k)",
                      "weight[(size_t)c * width + (width - 1 - k)] * XT(t - hist + k)"),
    "group_map": ("const int g = hd / heads_per_group;\n            const double *dtr",
                  "const int g = hd % ngroups;\n            const double *dtr"),
    "readout_before_update": ("y += Cr[(size_t)n * seqlen + t] * h[n];",
                              "y += Cr[(size_t)n * seqlen + t] * (h[n] - bx);"),
    "scan_delta_missing": ("const double bx = delta * Br[(size_t)n * seqlen + t] * ut;",
                           "const double bx = Br[(size_t)n * seqlen + t] * ut;"),
    "update_delta_missing": ("const double bx = delta * Bv[n] * xv;\n                    const double hn",
                             "const double bx = Bv[n] * xv;\n                    const double hn"),
    "skip_scaled": ("y += D[hd] * ut;", "y += D[hd] * ut * 0.5;"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "naive_softplus": ("return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));",
                       "return log(1.0 + exp(v));"),
    "tail_off_by_one": ("tail[j] = XT(seqlen - hist + j);", "tail[j] = XT(seqlen - hist + j - 1);"),
    "initial_state_ignored": ("h[n] = (st && has_initial_state) ? st[n] : 0.0;", "h[n] = 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_mutation(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "ssm_oracle.c"
    mut.write_text(text.replace(old, new))
    lib = tmp_path / "libssm_oracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", f"-I{ROOT}/oracle",
                           "-o", str(lib), str(mut), "-lm"])
    env = dict(os.environ, SSM_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins accepted the '{name}' mutation:\n{r.stdout[-2000:]}"
