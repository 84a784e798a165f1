"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/gdn_oracle.c, applies one plausible mistake (a dropped
term, a wrong sign, a transposed operand, a wrong index or convention),
compiles the copy on the CPU and runs tests/test_oracle_pins.py against it.
The pins must fail for every case.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    "no_decay": ("        S[i] *= a;", "        S[i] *= 1.0;"),
    "wrong_sign_of_prediction": ("d[j] = beta * (v[j] - p[j]);", "d[j] = beta * (v[j] + p[j]);"),
    "transposed_read": ("o[j] += S[i * dv + j] * q[i];", "o[j] += S[j * dv + i] * q[i];"),
    "read_before_write": ("    for (int j = 0; j < dv; ++j)\n        d[j] = beta * (v[j] - p[j]);",
                          "    for (int j = 0; j < dv; ++j)\n        d[j] = beta * (v[j] - p[j]);\n"
                          "    for (int j = 0; j < dv; ++j) { o[j] = 0.0; for (int i = 0; i < dk; ++i) o[j] += S[i * dv + j] * q[i]; }\n"
                          "    if (0)"),
    "eps_outside_root": ("double inv = scale / sqrt(ss + eps);", "double inv = scale / (sqrt(ss) + eps);"),
    "conv_taps_reversed": ("acc += w4[j] * xv;", "acc += w4[3 - j] * xv;"),
    "norm_one_plus_w": ("y[i] = w[i] * (o[i] * inv) * silu(z[i]);", "y[i] = (1.0 + w[i]) * (o[i] * inv) * silu(z[i]);"),
    "gqa_modulo": ("kh = h / ratio;", "kh = h % Hk;"),
    "no_query_scale": ("double sq_scale = 1.0 / sqrt((double)dk);", "double sq_scale = 1.0;"),
    "conv_state_newest_first": ("conv_state_in[((size_t)b * 3 + (size_t)(3 + tau)) * L->Cc + c]",
                                "conv_state_in[((size_t)b * 3 + (size_t)(-1 - tau)) * L->Cc + c]"),
    "chunk_output_strict_triangle": ("            for (int j = 0; j <= i; ++j) {\n                double qk = 0.0;",
                                     "            for (int j = 0; j < i; ++j) {\n                double qk = 0.0;"),
    "sigmoid_for_silu": ("static double silu(double x) { return x / (1.0 + exp(-x)); }",
                         "static double silu(double x) { return 1.0 / (1.0 + exp(-x)); }"),
    "norm_mean_over_sum": ("    ms /= (double)n;\n", "\n"),
    "gate_a_log_not_exponentiated": ("g[(size_t)t * Hv + h] = -exp(A_log[h]) * sp;",
                                     "g[(size_t)t * Hv + h] = -A_log[h] * sp;"),
    "gate_beta_wrong_sign": ("beta[(size_t)t * Hv + h] = 1.0 / (1.0 + exp(-b[(size_t)t * Hv + h]));",
                             "beta[(size_t)t * Hv + h] = 1.0 / (1.0 + exp(b[(size_t)t * Hv + h]));"),
    "gate_dt_bias_dropped": ("const double x = a[(size_t)t * Hv + h] + dt_bias[h];",
                             "const double x = a[(size_t)t * Hv + h];"),
    "gate_softplus_without_log": ("const double sp = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
                                  "const double sp = exp(x);"),
    "chunk_decay_not_relative": ("A[(size_t)i * n + j] = beta[t0 + i] * kk * exp(G[i] - G[j]);",
                                 "A[(size_t)i * n + j] = beta[t0 + i] * kk * exp(G[i]);"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-std=c11", "-shared", "-fPIC", "-o", str(lib), str(mut), "-lm"],
                   check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' passed every pin:\n{r.stdout[-2000:]}"
