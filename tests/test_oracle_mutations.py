"""Planted mistakes in a copy of the oracle must be caught by the pins.

Each case rewrites one expression of ``oracle/kda_oracle.c`` into a plausible
mistake (a dropped term, a wrong sign, a wrong operand or index), builds the
copy on the CPU, and runs ``test_oracle_pins.py`` against it in a child
process. The pins pass on the real oracle (their own test file) and must fail
on every mutant here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTANTS = {
    "decay_sign": ("double a = exp(gt[i]);", "double a = exp(-gt[i]);"),
    "delta_sign": ("u[j] = beta[t] * (vt[j] - sk);", "u[j] = beta[t] * (vt[j] + sk);"),
    "beta_dropped": ("u[j] = beta[t] * (vt[j] - sk);", "u[j] = (vt[j] - sk);"),
    "readout_uses_k": ("for (int32_t i = 0; i < K; ++i) s += S[(size_t)i * V + j] * qt[i];",
                       "for (int32_t i = 0; i < K; ++i) s += S[(size_t)i * V + j] * kt[i];"),
    "write_uses_q": ("S[(size_t)i * V + j] += kt[i] * u[j];", "S[(size_t)i * V + j] += qt[i] * u[j];"),
    "scale_dropped": ("o[(size_t)t * V + j] = scale * s;", "o[(size_t)t * V + j] = s;"),
    "softplus_sign": ("log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    "lb_no_A": ("return lower_bound * sigmoid(a * x);", "return lower_bound * sigmoid(x);"),
    "dt_bias_dropped": ("double x = raw_g + dt_bias;", "double x = raw_g;"),
    "beta_not_logistic": ("double kda_oracle_beta(double raw_beta) { return sigmoid(raw_beta); }",
                          "double kda_oracle_beta(double raw_beta) { return sigmoid(-raw_beta); }"),
    "bf16_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "q_from_k_block": ("q[(size_t)t * K + i] = kda_oracle_bf16_to_double(row[(size_t)h * K + i]);",
                       "q[(size_t)t * K + i] = kda_oracle_bf16_to_double(row[(size_t)H * K + (size_t)h * K + i]);"),
    "index_stride_ignored": ("a->state_indices[(int64_t)n * a->index_stride]", "a->state_indices[n]"),
    "chunk_P_no_diagonal": ("for (int32_t s = 0; s <= t; ++s) x += P[(size_t)t * C + s] * Vn[(size_t)s * V + j];",
                            "for (int32_t s = 0; s < t; ++s) x += P[(size_t)t * C + s] * Vn[(size_t)s * V + j];"),
    "chunk_state_no_decay": ("double x = exp(gl[i]) * S[(size_t)i * V + j];",
                             "double x = S[(size_t)i * V + j];"),
    "chunk_A_sign": ("A[(size_t)t * C + s] = (s < t) ? bc[t] * a : 0.0;",
                     "A[(size_t)t * C + s] = (s < t) ? -bc[t] * a : 0.0;"),
    "chunk_W_wrong_beta": ("x += Tm[(size_t)t * C + s] * bc[s] * kc[(size_t)s * K + i] *",
                           "x += Tm[(size_t)t * C + s] * bc[t] * kc[(size_t)s * K + i] *"),
    "chunk_cumsum_exclusive": ("acc += gc[(size_t)t * K + i];\n        gam[(size_t)t * K + i] = acc;",
                               "gam[(size_t)t * K + i] = acc;\n        acc += gc[(size_t)t * K + i];"),
    "spec_initial_column_fixed": ("const int64_t s0 = (int64_t)row[(int64_t)(acc - 1) * col_stride];",
                                  "const int64_t s0 = (int64_t)row[0];"),
    "spec_write_column_reversed": ("const int64_t st = (int64_t)row[(int64_t)t * col_stride];",
                                   "const int64_t st = (int64_t)row[(int64_t)(T - 1 - t) * col_stride];"),
    "spec_only_final_state_written": ("      if (st >= 0) {\n        float* tile",
                                      "      if (st >= 0 && t == T - 1) {\n        float* tile"),
    "norm_sum_not_mean": ("const double inv = 1.0 / sqrt(ss / V + eps);", "const double inv = 1.0 / sqrt(ss + eps);"),
    "norm_eps_outside_root": ("const double inv = 1.0 / sqrt(ss / V + eps);",
                              "const double inv = 1.0 / (sqrt(ss / V) + eps);"),
    "norm_gate_of_head_0": ("const uint16_t* zh = z + (size_t)r * z_row_stride + (size_t)h * V;",
                            "const uint16_t* zh = z + (size_t)r * z_row_stride;"),
    "norm_silu_as_sigmoid": ("const double act = activation == 1 ? zv * sigmoid(zv) : sigmoid(zv);",
                             "const double act = sigmoid(zv);"),
    "norm_weight_dropped": ("oh[j] = oh[j] * inv * (double)w[j] * act;", "oh[j] = oh[j] * inv * act;"),
    "conv_taps_reversed": ("a += (double)w[(size_t)c * W + i] * xv;", "a += (double)w[(size_t)c * W + (W - 1 - i)] * xv;"),
    "conv_history_off_by_one": (": hist[P + pos];\n          a +=", ": hist[P + pos - (pos > -P)];\n          a +="),
    "conv_sigmoid_not_silu": ("y[(size_t)(bos + t) * D + c] = a * sigmoid(a);", "y[(size_t)(bos + t) * D + c] = sigmoid(a);"),
    "conv_state_keeps_first_inputs": ("const int32_t pos = len - P + j;", "const int32_t pos = j;"),
    "conv_q_not_normalised": ("for (int32_t part = 0; part < 2; ++part)", "for (int32_t part = 1; part < 2; ++part)"),
    "conv_bias_dropped": ("double a = bias ? (double)bias[c] : 0.0;", "double a = 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_c = tmp_path / "kda_oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(so), str(mutant_c), "-lm"],
                   check=True)
    env = dict(os.environ, KDA_ORACLE_LIB_OVERRIDE=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"
    assert " failed" in r.stdout, r.stdout[-2000:]
