"""CPU pins of the oracle's static-P ablation (Shape.p_static): the forward's
P codes with the static scale s_P = 1/127 against the running maximum, the
alternative the SageAttention3 write-up names beside Eq. 8 and rejects as not
accurate enough (the method quantises P per token, s_P = exp(rowmax - m)/127)."""
import dataclasses

import numpy as np
import pytest

from oracle import fpa, metrics, sage
from tests.oracle_cases import gaussian_head


def _fwd(Q, K, V, sh, quant=True):
    qz = sage.quantize(Q, K, V, sh, quant)
    return sage.forward(qz, sh, quant)


def test_single_tile_static_equals_per_token():
    """With one key tile, every row's tile maximum is its running maximum:
    exp(rm - m)/127 = 1/127, so both scales and all codes coincide."""
    N, D = 64, 64
    Q, K, V, _ = gaussian_head(N, D, seed=82, sigma=2.0)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=64)
    O0, L0 = _fwd(Q, K, V, sh)
    O1, L1 = _fwd(Q, K, V, dataclasses.replace(sh, p_static=True))
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(L0, L1)


@pytest.mark.parametrize("causal", [False, True])
def test_quant_off_static_is_exact_attention(causal):
    N, D = 128, 32
    Q, K, V, _ = gaussian_head(N, D, seed=83, sigma=1.5)
    sh = sage.Shape(N=N, D=D, bq=32, bkv=32, causal=causal, k_smooth=False, p_static=True)
    O, L = _fwd(Q, K, V, sh, quant=False)
    O_ref, L_ref, _ = fpa.forward(Q, K, V, sh.scale, causal)
    np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L, L_ref, rtol=1e-10, atol=1e-12)


def test_static_scale_is_less_accurate():
    """The pages' reason for per-token scaling, against full-precision
    attention: on Gaussian heads the static scale is slightly worse; when one
    key of the first tile holds the running maximum of every row while the
    later tiles still carry most of the mass at lower logits, their
    probabilities get few of the 127 levels and the static scale is much
    worse."""
    N, D = 512, 64
    ratios = []
    for case in ("gaussian", "dominant"):
        Q, K, V, _ = gaussian_head(N, D, seed=84, sigma=1.0)
        if case == "dominant":
            u = np.ones(D) / np.sqrt(D)
            Q = Q + 2.0 * u[None, :]
            K[0] = 2.0 * np.sqrt(D) * u
        sh = sage.Shape(N=N, D=D, bq=64, bkv=64, k_smooth=False)
        O_ref, _, _ = fpa.forward(Q, K, V, sh.scale)
        e_tok = metrics.rel_l2(_fwd(Q, K, V, sh)[0], O_ref)
        e_sta = metrics.rel_l2(_fwd(Q, K, V, dataclasses.replace(sh, p_static=True))[0], O_ref)
        assert e_sta > e_tok, (case, e_tok, e_sta)
        ratios.append(e_sta / e_tok)
    assert ratios[1] > 1.4 and ratios[1] > ratios[0], ratios
