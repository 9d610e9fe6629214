"""The pins have teeth: each plausible mistake planted in a copy of the oracle
makes at least one pin fail.

Every mutant below is a one-line edit of one oracle source file
(oracle/mss_oracle.c for the scan, oracle/mss_oracle_conv.c for the conv1d,
oracle/mss_oracle_bwd.c for the scan's backward, oracle/mss_oracle_cplx.c for
the complex-A forward): a dropped term, a wrong
sign or index, a transposed or swapped operand, exp2 for exp, and so on.  The
altered copy is compiled, with the other sources as they are, into a
temporary library, and the pins of that source are run against it until one
fails; the real oracle sources are never modified.
"""

import os

import pytest

import oracle
import bwd_oracle_pins as BP
import conv_oracle_pins as CP
import cplx_oracle_pins as XP
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "mss_oracle.c")

MUTANTS = {
    "A_sign": ("A[n] = -exp(A_log[d * dstate + n]);", "A[n] = exp(A_log[d * dstate + n]);"),
    "A_no_exp": ("A[n] = -exp(A_log[d * dstate + n]);", "A[n] = -A_log[d * dstate + n];"),
    "decay_exp2": ("double a = exp(delta * A[n]);", "double a = exp2(delta * A[n]);"),
    "decay_no_delta": ("double a = exp(delta * A[n]);", "double a = exp(A[n]);"),
    "b_no_delta": ("double bt = delta * B_b[n * seqlen + t] * ut;",
                   "double bt = B_b[n * seqlen + t] * ut;"),
    "b_no_u": ("double bt = delta * B_b[n * seqlen + t] * ut;",
               "double bt = delta * B_b[n * seqlen + t];"),
    "b_uses_C": ("double bt = delta * B_b[n * seqlen + t] * ut;",
                 "double bt = delta * C_b[n * seqlen + t] * ut;"),
    "B_transposed": ("double bt = delta * B_b[n * seqlen + t] * ut;",
                     "double bt = delta * B_b[t * dstate + n] * ut;"),
    "B_time_shift": ("double bt = delta * B_b[n * seqlen + t] * ut;",
                     "double bt = delta * B_b[n * seqlen + (t > 0 ? t - 1 : 0)] * ut;"),
    "C_transposed": ("y += C_b[n * seqlen + t] * h[n];", "y += C_b[t * dstate + n] * h[n];"),
    "y_before_update": ("h[n] = a * h[n] + bt;\n                y += C_b[n * seqlen + t] * h[n];",
                        "y += C_b[n * seqlen + t] * h[n];\n                h[n] = a * h[n] + bt;"),
    "h_plus_not_times": ("h[n] = a * h[n] + bt;", "h[n] = a + h[n] + bt;"),
    "no_skip": ("y += skip * ut;", "y += 0.0 * skip * ut;"),
    "skip_uses_z": ("y += skip * ut;", "y += skip * (z_row ? z_row[t] : ut);"),
    "skip_after_gate": ("y += skip * ut;\n            if (z_row) y *= mss_oracle_silu(z_row[t]);",
                        "if (z_row) y *= mss_oracle_silu(z_row[t]);\n            y += skip * ut;"),
    "no_dt_bias": ("double x = delta_raw + bias;", "double x = delta_raw;"),
    "softplus_ignored": ("return delta_softplus ? mss_oracle_softplus(x) : x;", "return x;"),
    "softplus_always": ("return delta_softplus ? mss_oracle_softplus(x) : x;",
                        "return mss_oracle_softplus(x);"),
    "softplus_naive_log": ("return m + log1p(exp(-fabs(x)));", "return m + log(exp(-fabs(x)));"),
    "softplus_no_max": ("return m + log1p(exp(-fabs(x)));", "return log1p(exp(-fabs(x)));"),
    "gate_sigmoid_only": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "gate_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "h0_ignored": ("h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;", "h[n] = 0.0;"),
    "h0_transposed": ("h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;",
                      "h[n] = h0 ? h0[(b * dstate + n) * dim + d] : 0.0;"),
    "final_state_stale": ("final_state[(b * dim + d) * dstate + n] = h[n];",
                          "final_state[(b * dim + d) * dstate + n] = h[n] * 0.5;"),
    "step_decay_sign": ("double decay = exp(delta * -exp(A_log[d * dstate + n]));",
                        "double decay = exp(delta * exp(A_log[d * dstate + n]));"),
    "step_b_no_u": ("h[n] = decay * h[n] + delta * x * B[b * dstate + n];",
                    "h[n] = decay * h[n] + delta * B[b * dstate + n];"),
    "step_y_uses_B": ("y += h[n] * C[b * dstate + n];", "y += h[n] * B[b * dstate + n];"),
    "step_no_skip": ("y += (D ? D[d] : 0.0) * x;", "y += 0.0 * x;"),
    "step_no_bias": ("dt_bias ? dt_bias[d] : 0.0, delta_softplus);", "0.0, delta_softplus);"),
}

# conv1d mutants (oracle/mss_oracle_conv.c)
CONV_MUTANTS = {
    "conv_no_bias": ("double pre = bias ? bias[d] : 0.0;\n                for",
                     "double pre = 0.0;\n                for"),
    "conv_taps_reversed": ("pre += w_row[k] * extended_sample",
                           "pre += w_row[width - 1 - k] * extended_sample"),
    "conv_drop_current": ("for (int64_t k = 0; k < width; ++k)\n                    pre +=",
                          "for (int64_t k = 0; k + 1 < width; ++k)\n                    pre +="),
    "conv_window_shift": ("t - (width - 1) + k)", "t - (width - 1) + k - (t > 0))"),
    "conv_init_ignored": ("return init_row ? init_row[width - 1 + tau] : 0.0;", "return 0.0;"),
    "conv_init_reversed": ("return init_row ? init_row[width - 1 + tau] : 0.0;",
                           "return init_row ? init_row[-1 - tau] : 0.0;"),
    "conv_silu_ignored": ("out_row[t] = silu ? mss_oracle_silu(pre) : pre;", "out_row[t] = pre;"),
    "conv_final_shift": ("seqlen - (width - 1) + j);", "seqlen - width + j);"),
    "conv_step_no_shift": ("s[k] = window[k + 1];", "s[k] = window[k];"),
    "conv_step_taps_reversed": ("pre += w[d * width + k] * window[k];",
                                "pre += w[d * width + width - 1 - k] * window[k];"),
    "conv_step_x_dropped": ("window[width - 1] = x[b * dim + d];", "window[width - 1] = 0.0;"),
    "conv_step_no_bias": ("double pre = bias ? bias[d] : 0.0;\n            for",
                          "double pre = 0.0;\n            for"),
}
CONV_SRC = oracle.SOURCES["conv"]

# backward mutants (oracle/mss_oracle_bwd.c)
BWD_MUTANTS = {
    "bwd_no_dyC": ("double G = g[n] + dy * C_b[n * seqlen + t];", "double G = g[n];"),
    "bwd_dC_uses_prev": ("+= dy * h_t[n];", "+= dy * h_prev[n];"),
    "bwd_dB_no_delta": ("+= G * delta[t] * ut;", "+= G * ut;"),
    "bwd_da_uses_h_t": ("double ga = G * h_prev[n] * a;", "double ga = G * h_t[n] * a;"),
    "bwd_dA_log_sign": ("dA_log[d * dstate + n] += dA[n] * A[n];",
                        "dA_log[d * dstate + n] += -dA[n] * A[n];"),
    "bwd_g_no_decay": ("g[n] = G * a;", "g[n] = G;"),
    "bwd_no_softplus_grad": ("double dx = delta_softplus ? ddelta * sigmoid(x) : ddelta;",
                             "double dx = ddelta;"),
    "bwd_dz_no_y": ("dz[row + t] = dout[row + t] * y * silu_grad(z[row + t]);",
                    "dz[row + t] = dout[row + t] * silu_grad(z[row + t]);"),
    "bwd_silu_grad": ("return s * (1.0 + z * (1.0 - s));", "return s * (1.0 - s);"),
    "bwd_du_no_skip": ("double du_t = dy * skip;", "double du_t = 0.0;"),
    "bwd_dD_uses_dout": ("sum_dy_u += dy * ut;", "sum_dy_u += dout[row + t] * ut;"),
    "bwd_dfinal_ignored": ("g[n] = dfinal ? dfinal[(b * dim + d) * dstate + n] : 0.0;",
                           "g[n] = 0.0;"),
    "bwd_ddt_bias_raw": ("sum_dx += dx;", "sum_dx += ddelta;"),
    "bwd_ddelta_from_a_sign": ("ddelta += ga * A[n];", "ddelta -= ga * A[n];"),
}
BWD_SRC = oracle.SOURCES["bwd"]

CPLX_MUTANTS = {
    "cplx_imag_sign": ("-exp(A_log[d * dstate + n]) + I * A_imag[d * dstate + n];",
                       "-exp(A_log[d * dstate + n]) - I * A_imag[d * dstate + n];"),
    "cplx_real_no_exp": ("A[n] = -exp(A_log[d * dstate + n]) + I",
                         "A[n] = -A_log[d * dstate + n] + I"),
    "cplx_decay_modulus_only": ("double complex a = cexp(delta * A[n]);",
                                "double complex a = exp(delta * creal(A[n]));"),
    "cplx_decay_rotation_only": ("double complex a = cexp(delta * A[n]);",
                                 "double complex a = cexp(I * delta * cimag(A[n]));"),
    "cplx_decay_no_delta": ("double complex a = cexp(delta * A[n]);",
                            "double complex a = cexp(A[n]);"),
    "cplx_b_no_delta": ("double complex bt = delta * B[(b * dstate + n) * seqlen + t] * ut;",
                        "double complex bt = B[(b * dstate + n) * seqlen + t] * ut;"),
    "cplx_b_conj": ("double complex bt = delta * B[(b * dstate + n) * seqlen + t] * ut;",
                    "double complex bt = delta * conj(B[(b * dstate + n) * seqlen + t]) * ut;"),
    "cplx_h_conj": ("h[n] = a * h[n] + bt;", "h[n] = a * conj(h[n]) + bt;"),
    "cplx_C_conj": ("y += C[(b * dstate + n) * seqlen + t] * h[n];",
                    "y += conj(C[(b * dstate + n) * seqlen + t]) * h[n];"),
    "cplx_y_imag": ("double yr = creal(y) + skip * ut;", "double yr = cimag(y) + skip * ut;"),
    "cplx_y_modulus": ("double yr = creal(y) + skip * ut;", "double yr = cabs(y) + skip * ut;"),
    "cplx_no_skip": ("double yr = creal(y) + skip * ut;", "double yr = creal(y);"),
    "cplx_h0_ignored": ("h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;", "h[n] = 0.0;"),
    "cplx_no_gate": ("if (z) yr *= mss_oracle_silu(z[(b * dim + d) * seqlen + t]);", ""),
}
CPLX_SRC = oracle.SOURCES["cplx"]


def _run_pins(lib, pins=None, stop_at_first=False):
    failures = []
    for pin in pins if pins is not None else (P.ALL_PINS + CP.ALL_CONV_PINS + BP.ALL_BWD_PINS +
                                               XP.ALL_CPLX_PINS):
        try:
            pin(lib)
        except AssertionError as e:
            failures.append((pin.__name__, str(e)[:120]))
            if stop_at_first:
                break
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    oracle.build(str(mutated), str(so))
    # The library stays loaded: unloading a library whose OpenMP worker
    # threads are still parked is unsafe, and each mutant is small.
    failures = _run_pins(oracle.load(str(so)), P.ALL_PINS, stop_at_first=True)
    assert failures, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(name, tmp_path):
    old, new = CONV_MUTANTS[name]
    src = open(CONV_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutated = tmp_path / "mutant_conv.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    oracle.build(out=str(so), replace={"conv": str(mutated)})
    failures = _run_pins(oracle.load(str(so)), CP.ALL_CONV_PINS, stop_at_first=True)
    assert failures, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(BWD_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutated = tmp_path / "mutant_bwd.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    oracle.build(out=str(so), replace={"bwd": str(mutated)})
    failures = _run_pins(oracle.load(str(so)), BP.ALL_BWD_PINS, stop_at_first=True)
    assert failures, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(CPLX_MUTANTS))
def test_cplx_mutant_is_caught(name, tmp_path):
    old, new = CPLX_MUTANTS[name]
    src = open(CPLX_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutated = tmp_path / "mutant_cplx.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    oracle.build(out=str(so), replace={"cplx": str(mutated)})
    failures = _run_pins(oracle.load(str(so)), XP.ALL_CPLX_PINS, stop_at_first=True)
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "libcopy.so"
    oracle.build(SRC, str(so))
    assert _run_pins(oracle.load(str(so))) == []
