"""Pins of the accuracy metrics (oracle/metrics.py) against closed forms.

The SageAttention3 write-up defines cosine similarity, relative L1 and RMSE in
its table of quantisation-error metrics; the SageBwd listing's Tables 1 and 2
report cosine similarity and relative L2.  The GPU parity gate compares with
the cosine and the relative L2, so each metric is checked here on inputs whose
answer follows from the definition alone: identical, negated, orthogonal and
rescaled vectors, a fixed offset, a hand-worked three-element case, and the
zero-reference branches.
"""
import math

import numpy as np
import pytest

from oracle import metrics

RNG = np.random.default_rng(20260302)
X = RNG.standard_normal((7, 9))


def test_identical_tensors():
    m = metrics.all_metrics(X, X)
    assert m == {"cos": pytest.approx(1.0, abs=1e-15), "rel_l2": 0.0, "rel_l1": 0.0, "rmse": 0.0}


def test_negated_tensor():
    m = metrics.all_metrics(-X, X)
    assert m["cos"] == pytest.approx(-1.0, abs=1e-15)
    assert m["rel_l2"] == pytest.approx(2.0, rel=1e-15)
    assert m["rel_l1"] == pytest.approx(2.0, rel=1e-15)
    assert m["rmse"] == pytest.approx(2.0 * math.sqrt(np.mean(X * X)), rel=1e-14)


def test_orthogonal_vectors_have_zero_cosine():
    a = np.array([1.0, 2.0, 0.0, -3.0])
    b = np.array([2.0, -1.0, 5.0, 0.0])          # a . b = 0
    assert metrics.cos_sim(a, b) == 0.0
    assert metrics.rel_l2(a, b) == pytest.approx(math.sqrt(14 + 30) / math.sqrt(30), rel=1e-15)


@pytest.mark.parametrize("c", [0.25, 3.0, 1e6])
def test_positive_rescale(c):
    # cos ignores a positive factor; the relative errors of c * ref are |c - 1|
    assert metrics.cos_sim(c * X, X) == pytest.approx(1.0, abs=1e-15)
    assert metrics.rel_l2(c * X, X) == pytest.approx(abs(c - 1), rel=1e-12)
    assert metrics.rel_l1(c * X, X) == pytest.approx(abs(c - 1), rel=1e-12)


@pytest.mark.parametrize("e", [1e-3, -0.2, 0.5])
def test_relative_errors_of_a_proportional_perturbation(e):
    # x = ref (1 + e) elementwise: rel_l2 = rel_l1 = |e|, rmse = |e| rms(ref)
    x = X * (1 + e)
    assert metrics.rel_l2(x, X) == pytest.approx(abs(e), rel=1e-12)
    assert metrics.rel_l1(x, X) == pytest.approx(abs(e), rel=1e-12)
    assert metrics.rmse(x, X) == pytest.approx(abs(e) * math.sqrt(np.mean(X * X)), rel=1e-12)


def test_fixed_offset_rmse():
    assert metrics.rmse(X + 0.125, X) == pytest.approx(0.125, rel=1e-12)
    assert metrics.rmse(X - 3.0, X) == pytest.approx(3.0, rel=1e-12)


def test_hand_worked_three_elements():
    # x = (1, 2, 2), ref = (2, 0, 1): x . ref = 4, |x| = 3, |ref| = sqrt 5,
    # x - ref = (-1, 2, 1): |.|_2 = sqrt 6, |.|_1 = 4, sum |ref| = 3
    x = np.array([1.0, 2.0, 2.0])
    ref = np.array([2.0, 0.0, 1.0])
    assert metrics.cos_sim(x, ref) == pytest.approx(4 / (3 * math.sqrt(5)), rel=1e-15)
    assert metrics.rel_l2(x, ref) == pytest.approx(math.sqrt(6 / 5), rel=1e-15)
    assert metrics.rel_l1(x, ref) == pytest.approx(4 / 3, rel=1e-15)
    assert metrics.rmse(x, ref) == pytest.approx(math.sqrt(2), rel=1e-15)


def test_arguments_are_not_symmetric():
    # the second argument is the reference: relative errors divide by it
    x = np.array([1.0, 2.0, 2.0])
    ref = np.array([2.0, 0.0, 1.0])
    assert metrics.rel_l2(ref, x) == pytest.approx(math.sqrt(6) / 3, rel=1e-15)
    assert metrics.rel_l1(ref, x) == pytest.approx(4 / 5, rel=1e-15)


def test_zero_reference_branches():
    z = np.zeros(5)
    v = np.array([0.0, 3.0, 0.0, -4.0, 0.0])
    assert metrics.cos_sim(z, z) == 1.0           # both zero: identical
    assert metrics.cos_sim(v, z) == 0.0           # one zero: not identical
    assert metrics.rel_l2(v, z) == 5.0            # absolute norm when the reference is 0
    assert metrics.rel_l1(v, z) == 7.0
    assert metrics.rel_l2(z, z) == 0.0 and metrics.rel_l1(z, z) == 0.0
    assert metrics.rmse(np.zeros(0), np.zeros(0)) == 0.0


def test_shapes_are_flattened_and_computed_in_float64():
    a = X.astype(np.float32)
    b = (X * 1.001).astype(np.float32)
    flat = metrics.all_metrics(a.ravel(), b.ravel())
    assert metrics.all_metrics(a, b) == flat
    exact = np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b.astype(np.float64))
    assert flat["rel_l2"] == pytest.approx(exact, rel=1e-15)
