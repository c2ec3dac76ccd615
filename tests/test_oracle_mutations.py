"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutation edits one line of oracle/sage.py's (or oracle/metrics.py's)
source text, loads the edited copy as a separate module, swaps its functions
into ``oracle.sage`` (``oracle.metrics``) for the duration of the test, and
runs a few pins, at least one of which must fail.  Nothing here touches a GPU.
"""
import inspect
import sys
import types

import numpy as np
import pytest

import oracle.metrics as metrics_mod
import oracle.sage as sage_mod
from tests import test_oracle_bwd as tb
from tests import test_oracle_fp8 as tf8
from tests import test_oracle_fwd as tf
from tests import test_oracle_metrics as tm
from tests import test_oracle_quant as tq

SRC = inspect.getsource(sage_mod)
METRICS_SRC = inspect.getsource(metrics_mod)

MUTATIONS = {
    "drop_qsmooth_bias": ("S = S + qsmooth_bias(qz, i, j, sh)[None, :]", "S = S"),
    "no_alpha_rescale": ("acc = alpha[:, None] * acc + ", "acc = acc + "),
    "l_without_alpha": ("l = alpha * l + P_tilde.sum(axis=1)", "l = l + P_tilde.sum(axis=1)"),
    "ds_sign": ("dS = P * (dP - delta[rows][:, None])", "dS = P * (delta[rows][:, None] - dP)"),
    "dk_transposed": ("dK = (dS_hat.T @ qz.Qc[rows])", "dK = (dS_hat @ qz.Qc[rows])"),
    "dq_wrong_scale_index": ("(sdS * qz.sK[j])", "(sdS * qz.sK[i])"),
    "causal_strict": ("else (k <= q)", "else (k < q)"),
    "missing_dq_scale": ("return dQ * sh.scale, dK * sh.scale, dV", "return dQ, dK * sh.scale, dV"),
    "round_half_up": ("return np.clip(np.rint(x), lo, 127)", "return np.clip(np.floor(x + 0.5), lo, 127)"),
    "drop_dk_bias": ("dK[keys] += t[\"dK\"] + t[\"dKb\"]", "dK[keys] += t[\"dK\"]"),
    "kmean_over_block": ("mu_k = rnd(np.sum(K, axis=0) / N)", "mu_k = rnd(np.sum(K[:sh.bkv], axis=0) / sh.bkv)"),
    "p_scale_wrong_max": ("np.exp(rm - m_new))", "np.exp(m_new - rm))"),
    "dv_uses_p_not_codes": ("dV = (P_hat.T @ dOc[rows])", "dV = (P.T @ dOc[rows])"),
    "lse_log2": ("L[rows] = m + np.log(l)", "L[rows] = m + np.log2(l)"),
    "e4m3_no_subnormals": ("step = np.exp2(np.maximum(e - 1, -6) - 3)", "step = np.exp2((e - 1) - 3)"),
    "e4m3_ties_away": ("np.rint(x[nz] / step) * step   # exact scaling by a power of two, half-even",
                       "np.round(x[nz] / step + 1e-9) * step"),
    "e4m3_two_mantissa_bits": ("step = np.exp2(np.maximum(e - 1, -6) - 3)", "step = np.exp2(np.maximum(e - 1, -6) - 2)"),
    "fp8_block_scale_127": ("    qmax = 448 if fp8 else 127\n    x32", "    qmax = 127\n    x32"),
    "fp8_p_scale_127": ("    qmax = 448 if fp8 else 127\n    with", "    qmax = 127\n    with"),
}


def _mutated(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    return _load("oracle_sage_" + name, SRC.replace(old, new))


def _load(modname, text):
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod          # dataclasses look the module up by name
    try:
        exec(compile(text, "<" + modname + ">", "exec"), mod.__dict__)
    finally:
        del sys.modules[modname]
    return mod


PINS = [
    lambda: [tf.test_quant_off_forward_is_exact_attention(s, c, f) for s in tf.SHAPES[:2]
             for c in (False, True) for f in ((True, False), (True, True))],
    lambda: [tb.test_quant_off_backward_is_exact_gradient(c, f, b) for c in (False, True)
             for f in ((True, False), (True, True)) for b in ((64, 64), (32, 16))],
    lambda: tf.test_uniform_logits_average_values(True),
    lambda: tf.test_per_token_scale_is_static_value_at_row_max(),
    lambda: tf.test_online_recurrence_matches_two_pass(True, True),
    lambda: tb.test_uniform_probabilities_give_mean_dv(),
    lambda: tb.test_q_smoothing_quantised_dk_close_to_exact(),
    lambda: tb.test_q_smoothing_bias_restores_dk(),
    lambda: [tq.test_quantize_block_golden(c) for c in tq._read_golden()],
    lambda: tq.test_k_smoothing_centres_columns(),
    lambda: tf.test_quantised_forward_close_to_exact(),
    lambda: tf.test_per_token_codes_independent_of_running_max(),
    lambda: [tb.test_quantised_gradients_with_uneven_block_scales(c) for c in (False, True)],
    lambda: tf8.test_every_finite_encoding_round_trips(),
    lambda: tf8.test_rounding_matches_the_library_conversion(),
    lambda: tf8.test_block_codes_reach_448_and_stay_within_half_a_step(),
    lambda: tf8.test_forward_p_codes_top_out_at_448(),
]


def _catches(mod, target=sage_mod, pins=None):
    pins = PINS if pins is None else pins
    saved = {k: getattr(target, k) for k in dir(target) if not k.startswith("__")}
    try:
        for k in saved:
            if hasattr(mod, k):
                setattr(target, k, getattr(mod, k))
        caught = []
        for idx, pin in enumerate(pins):
            try:
                with np.errstate(all="ignore"):
                    pin()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(idx)
        return caught
    finally:
        for k, v in saved.items():
            setattr(target, k, v)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    assert _catches(_mutated(name)), f"no pin caught the planted mistake {name!r}"


def test_unmutated_copy_passes_all_pins():
    assert _catches(_load("oracle_sage_clean", SRC)) == []


# Mistakes in the metrics the GPU gate relies on (cosine and relative L2) and
# in the two reported ones.
METRIC_MUTATIONS = {
    "cos_numerator_self_dot": ("np.dot(a, b) / den", "np.dot(a, a) / den"),
    "cos_no_sqrt": ("den = np.sqrt(np.dot(a, a) * np.dot(b, b))", "den = np.dot(a, a) * np.dot(b, b)"),
    "cos_zero_branch": ("else float(np.array_equal(a, b))", "else 1.0"),
    "rel_l2_divides_by_x": ("np.linalg.norm(a - b) / nb)", "np.linalg.norm(a - b) / np.linalg.norm(a))"),
    "rel_l2_squared": ("np.linalg.norm(a - b) / nb)", "np.linalg.norm(a - b) ** 2 / nb)"),
    "rel_l1_abs_outside": ("np.sum(np.abs(a - b)) / sb", "np.abs(np.sum(a - b)) / sb"),
    "rel_l1_divides_by_x": ("sb = np.sum(np.abs(b))", "sb = np.sum(np.abs(a))"),
    "rmse_no_sqrt": ("np.sqrt(np.mean((a - b) ** 2))", "np.mean((a - b) ** 2)"),
    "rmse_sum": ("np.sqrt(np.mean((a - b) ** 2))", "np.sqrt(np.sum((a - b) ** 2))"),
}

METRIC_PINS = [getattr(tm, n) for n in dir(tm) if n.startswith("test_") and n not in (
    "test_positive_rescale", "test_relative_errors_of_a_proportional_perturbation")]
METRIC_PINS += [lambda: [tm.test_positive_rescale(c) for c in (0.25, 3.0)],
                lambda: [tm.test_relative_errors_of_a_proportional_perturbation(e) for e in (1e-3, -0.2)]]


@pytest.mark.parametrize("name", sorted(METRIC_MUTATIONS))
def test_metric_pins_catch_planted_mistake(name):
    old, new = METRIC_MUTATIONS[name]
    assert METRICS_SRC.count(old) == 1, name
    mod = _load("oracle_metrics_" + name, METRICS_SRC.replace(old, new))
    assert _catches(mod, metrics_mod, METRIC_PINS), f"no pin caught the planted mistake {name!r}"


def test_unmutated_metrics_pass_all_pins():
    assert _catches(_load("oracle_metrics_clean", METRICS_SRC), metrics_mod, METRIC_PINS) == []
