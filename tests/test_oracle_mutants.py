"""Plants plausible mistakes in the oracle's C source, one at a time, on the CPU, and checks that
the pin suite fails for every one of them (tests/test_oracle_pins.py for the forward and decode
step, tests/test_oracle_backward.py for the gradients). This is what makes the pins evidence: a
pin set that a slipped sign or a reversed tap survives would prove nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rglru_oracle.c")

MUTANTS = {
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    "softplus_arg": ("softplus(-lambda)", "softplus(lambda)"),
    "c_constant": ("#define RGLRU_ORACLE_C 8.0", "#define RGLRU_ORACLE_C 7.0"),
    "no_sqrt": ("double m = sqrt(1.0 - a * a);", "double m = (1.0 - a * a);"),
    "gates_swapped": ("double r = sigmoid(pa);\n  double ig = sigmoid(px);",
                      "double r = sigmoid(px);\n  double ig = sigmoid(pa);"),
    "no_decay_on_h": ("return a * h + m * (ig * xc);", "return h + m * (ig * xc);"),
    "no_input_gate": ("return a * h + m * (ig * xc);", "return a * h + m * xc;"),
    "conv_taps_reversed": ("acc += conv_w[(size_t)j * D + d] * xs[(size_t)s * D + d];",
                           "acc += conv_w[(size_t)(3 - j) * D + d] * xs[(size_t)s * D + d];"),
    "conv_halo_off_by_one": ("if (s >= 0) acc", "if (s > 0) acc"),
    "gate_matrix_transposed": ("const double *wa = W_a + ((size_t)g * Dh + o) * Dh;\n"
                               "          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;\n"
                               "          double sa = b_a[d], sx = b_x[d];\n"
                               "          for (int i = 0; i < Dh; ++i) {\n"
                               "            sa += wa[i] * xc[i];",
                               "const double *wa = W_a + ((size_t)g * Dh + o) * Dh;\n"
                               "          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;\n"
                               "          double sa = b_a[d], sx = b_x[d];\n"
                               "          for (int i = 0; i < Dh; ++i) {\n"
                               "            sa += W_a[((size_t)g * Dh + i) * Dh + o] * xc[i];"),
    "bias_dropped": ("double sa = b_a[d], sx = b_x[d];", "double sa = b_a[d], sx = 0.0;"),
    "y_is_previous_state": ("h[o] = rglru_step(h[o], xc[o], sa, sx, Lambda[d]);\n"
                            "          y[((size_t)b * T + t) * D + d] = h[o];",
                            "y[((size_t)b * T + t) * D + d] = h[o];\n"
                            "          h[o] = rglru_step(h[o], xc[o], sa, sx, Lambda[d]);"),
    "decode_state_reversed": ("acc += conv_w[(size_t)j * D + d] * cs[(size_t)j * D + d];",
                              "acc += conv_w[(size_t)j * D + d] * cs[(size_t)(K - 1 - j) * D + d];"),
    "decode_no_shift_in": ("cs[(size_t)(K - 1) * D + d] = xt[d];",
                           "cs[(size_t)(K - 1) * D + d] = 0.0;"),
}


# Mistakes in the backward (the forward it recomputes is shared with the forward above).
BACKWARD_MUTANTS = {
    "bwd_no_carry_decay": ("delta[o] = dl * a;", "delta[o] = dl;"),
    "bwd_normaliser_sign": ("dm * (-a * a / m)", "dm * (a * a / m)"),
    "bwd_dz_missing_a": ("double dz = da * a +", "double dz = da +"),
    "bwd_sigmoid_derivative": ("dpa[o] = dr * r * (1.0 - r);", "dpa[o] = dr * r;"),
    "bwd_dlambda_sign": ("dLambda[d] += -sigmoid(-Lambda[d]) * dsp;",
                         "dLambda[d] += sigmoid(-Lambda[d]) * dsp;"),
    "bwd_dW_transposed": ("gwa[i] += dpa[o] * xc[(size_t)t * Dh + i];",
                          "gwa[i] += dpa[i] * xc[(size_t)t * Dh + o];"),
    "bwd_drops_input_gate_path": ("dxc[(size_t)t * Dh + i] += wa[i] * dpa[o] + wx[i] * dpx[o];",
                                  "dxc[(size_t)t * Dh + i] += wa[i] * dpa[o];"),
    "bwd_conv_taps_reversed": ("dx[((size_t)b * T + s) * D + d] += conv_w[(size_t)j * D + d]",
                               "dx[((size_t)b * T + s) * D + d] += conv_w[(size_t)(K - j) * D + d]"),
    "bwd_state_off_by_one": ("double hprev = t > 0 ? hs[(size_t)(t - 1) * Dh + o]",
                             "double hprev = t > 0 ? hs[(size_t)t * Dh + o]"),
    "bwd_ignores_dh_T": ("delta[o] = dh_T ? dh_T[(size_t)b * D + g * Dh + o] : 0.0;",
                         "delta[o] = 0.0;"),
}


def _run_mutant(name, old, new, pins, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(mutant), "-lm"], check=True)
    env = dict(os.environ, RGLRU_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", pins)],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    _run_mutant(name, *MUTANTS[name], "test_oracle_pins.py", tmp_path)


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    _run_mutant(name, *BACKWARD_MUTANTS[name], "test_oracle_backward.py", tmp_path)
