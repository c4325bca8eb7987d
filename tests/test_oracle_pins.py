"""The oracle against its pins, and every pin set against planted mistakes.

A mutant is a copy of the oracle's C source with one plausible mistake
written in (a dropped term, a wrong sign, a wrong operand, a misplaced read).
Each must fail at least one pin; the unmodified oracle must pass all of them.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
from tests import oracle_pins



@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.Oracle())


SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, text in kda_oracle.c, replacement)
MUTANTS = [
    ("no_fade", "S[c * V + j] *= at[c];", "(void)at;"),
    ("fade_by_value_col", "S[c * V + j] *= at[c];", "S[c * V + j] *= at[j % K];"),
    ("accumulate_only", "bt * kt[c] * (vt[j] - pred[j])", "bt * kt[c] * vt[j]"),
    ("wrong_sign", "S[c * V + j] += bt * kt[c] * (vt[j] - pred[j]);",
     "S[c * V + j] -= bt * kt[c] * (vt[j] - pred[j]);"),
    ("predict_with_query", "pred[j] += S[c * V + j] * kt[c];", "pred[j] += S[c * V + j] * qt[c];"),
    ("no_beta", "bt * kt[c] * (vt[j] - pred[j])", "kt[c] * (vt[j] - pred[j])"),
    ("read_before_write",
     "/* correct: S += beta_t * k_t (v_t - prediction)^T */",
     "/* correct moved */ { double *ot0 = out + (t * H + h) * V; for (int64_t j = 0; j < V; ++j) { double a0 = 0.0; for (int64_t c = 0; c < K; ++c) a0 += S[c * V + j] * qt[c]; ot0[j] = scale * a0; } }"),
    ("read_ignores_scale", "ot[j] = scale * acc;", "ot[j] = acc;"),
    ("initial_state_ignored", "if (s0)\n        memcpy", "if (0)\n        memcpy"),
    ("gate_scale_outside", "double g = g_min * sigmoid(scale * x);", "double g = g_min * scale * sigmoid(x);"),
    ("gate_log_scale_not_exp", "double scale = exp(log_scale[h]);", "double scale = log_scale[h];"),
    ("gate_no_bias", "double x = z[i] + (bias ? bias[h * K + c] : 0.0);", "double x = z[i];"),
    ("gate_softplus", "double g = g_min * sigmoid(scale * x);", "double g = -scale * log1p(exp(x));"),
    ("gate_returns_log", "out[i] = out_log ? g : exp(g);", "out[i] = g;"),
    # mistakes in the gradients
    ("bwd_no_fade_chain", "dS[c * V + j] = at[c] * dP[c * V + j];", "dS[c * V + j] = dP[c * V + j];"),
    ("bwd_dk_drops_prediction", "dk[(t * H + h) * K + c] -= acc;", "(void)acc;"),
    ("bwd_dq_no_scale", "dq[(t * H + h) * K + c] = scale * acc;", "dq[(t * H + h) * K + c] = acc;"),
    ("bwd_dbeta_sign", "db += kt[c] * acc;", "db -= kt[c] * acc;"),
    ("bwd_dv_no_beta", "dd[j] = bt * acc;", "dd[j] = acc;"),
    ("bwd_dalpha_new_state", "acc += dP[c * V + j] * Sprev[c * V + j];", "acc += dP[c * V + j] * Scur[c * V + j];"),
    ("bwd_read_with_key", "dS[c * V + j] += scale * qt[c] * dot[j];", "dS[c * V + j] += scale * kt[c] * dot[j];"),
    ("bwd_dP_no_correction", "dP[c * V + j] = dS[c * V + j] - kt[c] * dd[j];", "dP[c * V + j] = dS[c * V + j];"),
    ("bwd_final_grad_ignored", "if (dsT)\n        memcpy(dS, dsT", "if (0)\n        memcpy(dS, dsT"),
    ("bwd_delta_undecayed", "acc += at[c] * Sprev[c * V + j] * kt[c];", "acc += Sprev[c * V + j] * kt[c];"),
    ("gate_bwd_no_exp_scale", "dz[i] = dx * e;", "dz[i] = dx;"),
    ("gate_bwd_log_scale_no_x", "dlog_scale[h] += dx * x;", "dlog_scale[h] += dx;"),
    ("gate_bwd_no_alpha_factor", "grad[i] * exp(g)", "grad[i]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor missing: %s" % name
    if name == "read_before_write":
        # the read happens before the correction; the later read is removed
        src = src.replace(old, new, 1)
        src = src.replace("ot[j] = scale * acc;", "(void)acc; (void)ot;", 1)
    else:
        src = src.replace(old, new, 1)
    msrc = tmp_path / ("mut_%s.c" % name)
    msrc.write_text(src)
    lib = oracle.compile_oracle(str(msrc), str(tmp_path / ("mut_%s.so" % name)))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
