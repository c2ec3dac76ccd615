"""CPU pins of QK-norm fused into the oracle's preprocessing (Shape.qk_norm):
per-token RMS normalisation of Q and K (unit gain, eps 1e-6) before smoothing
and quantisation, and the gradients passed back through it."""
import dataclasses

import numpy as np
import pytest

from oracle import fpa, sage
from tests.oracle_cases import gaussian_head


def test_normalised_rows_have_unit_rms():
    """Closed form: mean(x_n^2) = ms / (ms + eps) for each row."""
    X = gaussian_head(64, 128, seed=101, sigma=3.0)[0]
    Xn, r = sage.rms_norm(X, quant=True)
    ms = np.mean(X * X, axis=1)
    np.testing.assert_allclose(np.mean(Xn * Xn, axis=1), ms / (ms + sage.QK_NORM_EPS), rtol=3e-7)
    assert r.dtype == np.float64 and np.all(r.astype(np.float32) == r)


@pytest.mark.parametrize("causal", [False, True])
def test_quant_off_gradients_through_the_norm_match_finite_differences(causal):
    """f(Q, K, V) = sum(O(norm(Q), norm(K), V) o dO): central differences of
    the textbook attention of the normalised rows against the oracle's
    chain-rule gradients with quantisation off."""
    N, D = 32, 8
    Q, K, V, dO = gaussian_head(N, D, seed=102, sigma=2.0)
    sh = sage.Shape(N=N, D=D, bq=16, bkv=16, causal=causal, qk_norm=True)
    r = sage.run_head(Q, K, V, dO, sh, quant=False)

    def f(Qx, Kx):
        qn = Qx / np.sqrt(np.mean(Qx * Qx, axis=1, keepdims=True) + sage.QK_NORM_EPS)
        kn = Kx / np.sqrt(np.mean(Kx * Kx, axis=1, keepdims=True) + sage.QK_NORM_EPS)
        return np.sum(fpa.forward(qn, kn, V, sh.scale, causal)[0] * dO)

    h = 1e-6
    for name, X, grad in (("Q", Q, r["dQ_in"]), ("K", K, r["dK_in"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            num[idx] = (f(Xp, K) - f(Xm, K)) / (2 * h) if name == "Q" else (f(Q, Xp) - f(Q, Xm)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_norm_backward_is_orthogonal_to_the_row():
    """The normalised output does not change when a row is scaled, so the
    input gradient of each row is orthogonal to that row (up to eps):
    sum_d x_d * dL/dx_d = r * eps / (ms + eps) * sum(dX_n o X) ~ 0."""
    X = gaussian_head(32, 64, seed=103, sigma=2.0)[0]
    g = gaussian_head(32, 64, seed=104)[0]
    _, r = sage.rms_norm(X, quant=False)
    dX = sage.rms_norm_backward(X, r, g, quant=False)
    dots = np.sum(dX * X, axis=1)
    assert np.max(np.abs(dots)) < 1e-5 * np.max(np.abs(np.sum(g * X, axis=1)))
