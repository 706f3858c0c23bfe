"""Plant plausible mistakes in copies of the oracle and check the pins catch
every one of them.

Each mutant is the oracle's C source with one textual change, compiled with
gcc into a temporary directory (CPU only).  The pin tests of
``test_oracle_pins`` are then run against the mutant; at least one must fail.
This shows the pins constrain every step of the recurrence (fade, predict,
correct, read, scale, state hand-over, the delta switch), not only its shape.
"""
import os

import pytest

import test_oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "kda_oracle.c")

_CORRECT_READ = """    /* 3. correct: write the residual v_t - prediction along k_t, strength beta_t. */
    for (j = 0; j < dv; ++j) tmp[j] = v[j] - tmp[j];
    for (i = 0; i < dk; ++i) {
        const double bk = beta * k[i];
        double *row = S + i * dv;
        for (j = 0; j < dv; ++j) row[j] += bk * tmp[j];
    }
"""
_FADE = """    for (i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        double *row = S + i * dv;
        for (j = 0; j < dv; ++j) row[j] *= a;
    }
"""

_READ = """    /* 4. read the state after this token's write. */
    if (o) {
        for (j = 0; j < dv; ++j) tmp[j] = 0.0;
        for (i = 0; i < dk; ++i) {
            const double qi = q[i];
            const double *row = S + i * dv;
            for (j = 0; j < dv; ++j) tmp[j] += row[j] * qi;
        }
        for (j = 0; j < dv; ++j) o[j] = scale * tmp[j];
    }
"""

MUTANTS = {
    "readout_before_write": (_READ, ""),
    "fade_with_inverse_decay": ("const double a = exp(g[i]);", "const double a = exp(-g[i]);"),
    "fade_dropped": ("const double a = exp(g[i]);", "const double a = 1.0;"),
    "fade_on_value_columns": ("for (j = 0; j < dv; ++j) row[j] *= a;",
                              "for (j = 0; j < dv; ++j) row[j] *= exp(g[j % dk]);"),
    "fade_after_write": (_FADE + "    /* 2.", "    /* 2."),
    "residual_sign_flipped": ("tmp[j] = v[j] - tmp[j];", "tmp[j] = v[j] + tmp[j];"),
    "beta_dropped": ("const double bk = beta * k[i];", "const double bk = k[i];"),
    "key_dropped_from_write": ("const double bk = beta * k[i];", "const double bk = beta;"),
    "prediction_uses_query": ("for (j = 0; j < dv; ++j) tmp[j] += row[j] * ki;",
                              "for (j = 0; j < dv; ++j) tmp[j] += row[j] * q[i];"),
    "readout_not_transposed": ("for (j = 0; j < dv; ++j) tmp[j] += row[j] * qi;",
                               "for (j = 0; j < dv; ++j) tmp[j] += (j < dk && i < dv ? S[j * dv + i] : 0.0) * qi;"),
    "readout_scale_dropped": ("o[j] = scale * tmp[j];", "o[j] = tmp[j];"),
    "initial_state_ignored": ("if (S0) memcpy(S, S0", "if (0) memcpy(S, S0"),
    "delta_always_on": ("if (delta) {", "if (1) {"),
    "delta_always_off": ("if (delta) {", "if (0) {"),
    # backward (reverse-mode adjoint of the token recurrence)
    "bwd_readout_gradient_dropped": ("for (j = 0; j < dv; ++j) dS[i * dv + j] += scale * q[i] * dout[j];",
                                     "for (j = 0; j < dv; ++j) (void)dout[j];"),
    "bwd_dq_scale_dropped": ("dq[i] = scale * acc;", "dq[i] = acc;"),
    "bwd_dbeta_sign_flipped": ("*dbeta = acc;", "*dbeta = -acc;"),
    "bwd_dv_sign_flipped": ("dval[j] = beta * w[j];", "dval[j] = -beta * w[j];"),
    "bwd_dk_prediction_term_dropped": ("dkey[i] += acc;", "dkey[i] += 0.0 * acc;"),
    "bwd_state_prediction_term_dropped": ("dS[i * dv + j] += k[i] * dp[j];   /* dS is now dD */",
                                          "(void)dp[j];"),
    "bwd_dg_from_undecayed_state": ("acc += D[i * dv + j] * dS[i * dv + j];",
                                    "acc += S_prev[i * dv + j] * dS[i * dv + j];"),
    "bwd_state_gradient_not_faded": ("for (j = 0; j < dv; ++j) dS[i * dv + j] *= alpha;", "(void)alpha;"),
    "bwd_segment_recompute_off_by_one": ("const int64_t th = (a0 + t - 1) * H + h;",
                                         "const int64_t th = (a0 + t) * H + h;"),
    "bwd_final_state_gradient_ignored": ("if (dS_T) memcpy(dS, dS_T", "if (0) memcpy(dS, dS_T"),
    "bwd_initial_state_ignored": ("if (S0) memcpy(dS, S0", "if (0) memcpy(dS, S0"),
}


def _apply(src, name):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    out = src.replace(old, new)
    if name == "fade_after_write":
        # the fade block moves after the correction, before the readout
        out = out.replace(_CORRECT_READ, _CORRECT_READ + _FADE)
        assert out.count(_FADE) == 1
    if name == "readout_before_write":
        # the readout moves ahead of the prediction (it then sees D S_{t-1})
        out = out.replace("    /* 2. predict", _READ + "    /* 2. predict")
        assert out.count(_READ) == 1
    return out


PIN_CALLS = [
    ("p1", lambda m: pins.test_p1_worked_delta_example(m)),
    ("p2", lambda m: pins.test_p2_exact_recall_after_write(m, 5, 3)),
    ("p3", lambda m: pins.test_p3_linear_attention_double_sum(m)),
    ("p3b", lambda m: pins.test_p3b_gated_linear_closed_form(m)),
    ("p4", lambda m: pins.test_p4_pure_decay_rows(m)),
    ("p5", lambda m: pins.test_p5_equivalent_forms(m, "product")),
    ("p6", lambda m: pins.test_p6_brute_force_unrolled_packed(m)),
    ("p7", lambda m: pins.test_p7_toy_demo_printed_errors(m)),
    ("p9", lambda m: pins.test_p9_superposition(m)),
    ("p14", lambda m: pins.test_p14_backward_finite_differences(m, 2)),
    ("p15", lambda m: pins.test_p15_backward_matches_autograd(m)),
]


def test_unmutated_copy_passes_every_pin(tmp_path):
    import oracle
    src = open(ORACLE_SRC).read()
    path = tmp_path / "copy.c"
    path.write_text(src)
    lib = oracle.OracleLib(oracle.compile_source(str(path), str(tmp_path / "libcopy.so")))
    for _, call in PIN_CALLS:
        call(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    import oracle
    src = _apply(open(ORACLE_SRC).read(), name)
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src)
    lib = oracle.OracleLib(oracle.compile_source(str(path), str(tmp_path / ("lib%s.so" % name))))
    caught = []
    for pin, call in PIN_CALLS:
        try:
            call(lib)
        except (AssertionError, ValueError):
            caught.append(pin)
    assert caught, "mutant %s passed every pin" % name
