"""CPU pins of the oracle's forward pass."""
import numpy as np
import pytest
import torch

from oracle import fpa, sage
from tests.oracle_cases import gaussian_head

SHAPES = [
    dict(N=128, D=32, bq=64, bkv=64),
    dict(N=256, D=64, bq=128, bkv=64),
    dict(N=96, D=16, bq=32, bkv=16),
]


def _sdpa_forward(Q, K, V, scale, causal):
    q, k, v = (torch.tensor(a)[None, None] for a in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_fpa_matches_torch_sdpa(causal):
    Q, K, V, _ = gaussian_head(96, 16, seed=1, sigma=2.0)
    O, L, P = fpa.forward(Q, K, V, 0.25, causal)
    np.testing.assert_allclose(O, _sdpa_forward(Q, K, V, 0.25, causal), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-14)
    S = (Q @ K.T) * 0.25
    if causal:
        S = np.where(fpa.causal_mask(96, 96), S, -np.inf)
    np.testing.assert_allclose(L, np.log(np.sum(np.exp(S), axis=1)), rtol=1e-13)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("smooth", [(True, False), (False, False), (True, True)])
def test_quant_off_forward_is_exact_attention(shape, causal, smooth):
    N, D = shape["N"], shape["D"]
    Q, K, V, _ = gaussian_head(N, D, seed=N + D, sigma=1.5, k_offset=2.0, q_offset=1.0)
    sh = sage.Shape(**shape, causal=causal, k_smooth=smooth[0], q_smooth=smooth[1])
    qz = sage.quantize(Q, K, V, sh, quant=False)
    O, L = sage.forward(qz, sh, quant=False)
    O_ref, L_ref, _ = fpa.forward(Q, K, V, sh.scale, causal)
    np.testing.assert_allclose(O, O_ref, rtol=1e-11, atol=1e-12)
    # L is the logsumexp of the logits the kernel forms, i.e. of Q (K - mu_K)^T:
    # K-smoothing shifts each row by -scale * q . mu_K (O does not move).
    np.testing.assert_allclose(L, L_ref - sh.scale * (Q @ qz.mu_k), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_smooth", [False, True])
def test_online_recurrence_matches_two_pass(causal, q_smooth):
    Q, K, V, _ = gaussian_head(256, 64, seed=21, sigma=2.0, k_offset=1.0, q_offset=1.0)
    sh = sage.Shape(N=256, D=64, bq=64, bkv=32, causal=causal, q_smooth=q_smooth)
    qz = sage.quantize(Q, K, V, sh)
    O1, L1 = sage.forward(qz, sh)
    O2, L2 = sage.forward_two_pass(qz, sh)
    np.testing.assert_array_equal(L1, L2)
    # identical codes; O differs only by float64 rounding before the bf16 rounding
    diff = np.abs(O1 - O2)
    assert np.mean(diff > 0) < 1e-3
    assert np.all(diff <= np.abs(O2) * 2 ** -7 + 1e-30)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_logits_average_values(causal):
    """Q = 0 makes every logit 0: P~ = 1, every P code 127, and O is the mean of
    the visible V rows (V integer-valued with 127 in every block, so V^ = V)."""
    N, D = 128, 16
    rng = np.random.default_rng(5)
    V = rng.integers(-120, 121, size=(N, D)).astype(np.float64)
    V[::32, 0] = 127.0
    Q = np.zeros((N, D)); K = rng.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, causal=causal, dtype=1)
    qz = sage.quantize(Q, K, V, sh)
    assert np.all(qz.sV == 1.0) and np.array_equal(qz.Vc, V)
    O, L = sage.forward(qz, sh)
    if causal:
        mean = np.cumsum(V, axis=0) / np.arange(1, N + 1)[:, None]
        lse = np.log(np.arange(1, N + 1))
    else:
        mean = np.tile(V.mean(axis=0), (N, 1))
        lse = np.full(N, np.log(N))
    # the only error besides bf16 rounding is 127 * f32(1/127) != 1 (4e-9)
    assert np.all(np.abs(O - mean) <= np.abs(mean) * 2 ** -8 + 1e-12)
    np.testing.assert_allclose(L, lse, rtol=1e-7)


def test_per_token_scale_is_static_value_at_row_max():
    """Where the tile's row max is the running max, s_P = 1/127 in float32 and
    the max element's code is 127 (SA3 Eq. 8)."""
    P_tilde = np.array([[1.0, 0.5, 0.25, 0.0], [1.0, 1.0, 0.999, 0.001]])
    rm = np.zeros(2); m_new = np.zeros(2)
    sP, codes = sage.per_token_p_quant(P_tilde, rm, m_new)
    assert np.all(sP == float(np.float32(1) / np.float32(127)))
    assert codes.tolist() == [[127, 64, 32, 0], [127, 127, 127, 0]]
    # a fully masked row in this tile: scale 0, codes 0
    sP, codes = sage.per_token_p_quant(np.zeros((1, 4)), np.array([-np.inf]), np.array([0.3]))
    assert sP[0] == 0 and not codes.any()


def test_per_token_codes_independent_of_running_max():
    """P~ / s_P = 127 exp(S - rowmax), whatever the running max is."""
    rng = np.random.default_rng(9)
    S = rng.standard_normal((8, 64)) * 3
    rm = S.max(axis=1)
    for shift in (0.0, 0.7, 5.0):
        m_new = rm + shift
        P_tilde = np.exp(S - m_new[:, None])
        _, codes = sage.per_token_p_quant(P_tilde, rm, m_new)
        exact = 127 * np.exp(S - rm[:, None])
        clear = np.abs(exact - np.floor(exact) - 0.5) > 1e-4
        assert np.array_equal(codes[clear], np.rint(exact)[clear])


def test_k_smoothing_leaves_quant_off_output_unchanged():
    Q, K, V, _ = gaussian_head(128, 32, seed=8, k_offset=5.0)
    outs = []
    for ks in (False, True):
        sh = sage.Shape(N=128, D=32, bq=64, bkv=64, k_smooth=ks, causal=True)
        outs.append(sage.forward(sage.quantize(Q, K, V, sh, quant=False), sh, quant=False))
    np.testing.assert_allclose(outs[0][0], outs[1][0], rtol=1e-11, atol=1e-12)


def test_k_smoothing_reduces_quantised_error_with_offset_keys():
    """K-smoothing is what keeps the INT8 logits accurate when K carries a
    large per-channel offset (paperlayer section 6; SA3 smoothing ablation)."""
    Q, K, V, _ = gaussian_head(256, 64, seed=12, k_offset=8.0)
    errs = {}
    for ks in (False, True):
        sh = sage.Shape(N=256, D=64, bq=128, bkv=64, k_smooth=ks)
        O, _ = sage.forward(sage.quantize(Q, K, V, sh), sh)
        O_ref, _, _ = fpa.forward(Q, K, V, sh.scale)
        errs[ks] = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    assert errs[True] < 0.5 * errs[False]
    assert errs[True] < 0.05


def test_quantised_forward_close_to_exact():
    Q, K, V, _ = gaussian_head(256, 128, seed=13)
    sh = sage.Shape(N=256, D=128, bq=128, bkv=64)
    qz = sage.quantize(Q, K, V, sh)
    O, L = sage.forward(qz, sh)
    O_ref, L_ref, _ = fpa.forward(Q, K, V, sh.scale)
    rel = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    assert 1e-4 < rel < 0.05
    np.testing.assert_allclose(L, L_ref - sh.scale * (Q @ qz.mu_k), atol=0.05)
