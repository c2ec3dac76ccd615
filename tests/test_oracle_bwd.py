"""CPU pins of the oracle's backward pass."""
import numpy as np
import pytest
import torch

from oracle import fpa, sage
from tests.oracle_cases import gaussian_head


def _torch_grads(Q, K, V, dO, scale, causal):
    q, k, v = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                                         is_causal=causal, scale=scale)[0, 0]
    o.backward(torch.tensor(dO))
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _full(Q, K, V, dO, sh, quant):
    qz = sage.quantize(Q, K, V, sh, quant)
    O, L = sage.forward(qz, sh, quant)
    delta, dOc, sdO = sage.backward_pre(O, dO, sh, quant)
    dQ, dK, dV = sage.backward(qz, V, dO, dOc, sdO, L, delta, sh, quant)
    return qz, O, L, delta, dOc, sdO, dQ, dK, dV


@pytest.mark.parametrize("causal", [False, True])
def test_fpa_gradients_match_torch_autograd(causal):
    Q, K, V, dO = gaussian_head(64, 16, seed=2, sigma=1.5)
    g = fpa.backward(Q, K, V, dO, 0.3, causal)
    tq, tk, tv = _torch_grads(Q, K, V, dO, 0.3, causal)
    np.testing.assert_allclose(g["dQ"], tq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dK"], tk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dV"], tv, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("flags", [(True, False), (False, False), (True, True)])
def test_quant_off_gradients_match_finite_differences(causal, flags):
    """Central differences of f = sum(O o dO) w.r.t. every entry of Q, K, V."""
    N, D = 32, 8
    Q, K, V, dO = gaussian_head(N, D, seed=31, k_offset=1.0, q_offset=1.0)
    sh = sage.Shape(N=N, D=D, bq=16, bkv=8, causal=causal, k_smooth=flags[0], q_smooth=flags[1])
    *_, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=False)

    def f(Qx, Kx, Vx):
        O, _ = sage.forward(sage.quantize(Qx, Kx, Vx, sh, quant=False), sh, quant=False)
        return np.sum(O * dO)

    h = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("flags", [(True, False), (False, False), (True, True)])
@pytest.mark.parametrize("blocks", [(64, 64), (128, 64), (32, 16)])
def test_quant_off_backward_is_exact_gradient(causal, flags, blocks):
    N, D = 256, 32
    Q, K, V, dO = gaussian_head(N, D, seed=40, sigma=1.3, k_offset=2.0, q_offset=1.5)
    sh = sage.Shape(N=N, D=D, bq=blocks[0], bkv=blocks[1], causal=causal, k_smooth=flags[0], q_smooth=flags[1])
    *_, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=False)
    g = fpa.backward(Q, K, V, dO, sh.scale, causal)
    for ours, ref in ((dQ, g["dQ"]), (dK, g["dK"]), (dV, g["dV"])):
        np.testing.assert_allclose(ours, ref, rtol=1e-9, atol=1e-11)


def test_delta_identity_and_row_sums():
    """rowsum(dO o O) = rowsum(P o dP), hence every row of dS sums to 0
    (quantisation off)."""
    N, D = 128, 32
    Q, K, V, dO = gaussian_head(N, D, seed=41, k_offset=2.0)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, causal=True)
    qz, O, L, delta, dOc, sdO, *_ = _full(Q, K, V, dO, sh, quant=False)
    P = np.zeros((N, N)); dP = np.zeros((N, N)); dS = np.zeros((N, N))
    for i in range(sh.Tm):
        for j in range(sh.Tn):
            if not sage.tile_visible(i, j, sh):
                continue
            t = sage.backward_tile(qz, V, dO, dOc, sdO, L, delta, i, j, sh, quant=False)
            r, c = slice(i * 64, (i + 1) * 64), slice(j * 32, (j + 1) * 32)
            P[r, c], dP[r, c], dS[r, c] = t["P"], t["dP"], t["dS"]
    np.testing.assert_allclose(delta, np.sum(P * dP, axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dS.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("quant", [False, True])
def test_ds_magnitude_bound(quant):
    """SageBwd appendix B: per row, RMS(dS_i) <= max_n |dP_in - delta_i| / sqrt(N)."""
    N, D = 256, 64
    Q, K, V, dO = gaussian_head(N, D, seed=42, sigma=2.0)
    sh = sage.Shape(N=N, D=D, bq=128, bkv=64)
    qz, O, L, delta, dOc, sdO, *_ = _full(Q, K, V, dO, sh, quant=quant)
    dS = np.zeros((N, N)); dP = np.zeros((N, N))
    for i in range(sh.Tm):
        for j in range(sh.Tn):
            t = sage.backward_tile(qz, V, dO, dOc, sdO, L, delta, i, j, sh, quant=quant)
            r, c = slice(i * 128, (i + 1) * 128), slice(j * 64, (j + 1) * 64)
            dS[r, c], dP[r, c] = t["dS"], t["dP"]
    rms = np.sqrt(np.mean(dS ** 2, axis=1))
    bound = np.max(np.abs(dP - delta[:, None]), axis=1) / np.sqrt(N)
    assert np.all(rms <= bound * (1 + 1e-5))
    assert np.median(rms / bound) < 0.5     # the bound is not vacuous either way


def test_dp_is_unquantised():
    """Table 2 of the SageBwd paper lists dP with cosine 1.0000 and rel-L2
    0.0000: dP = dO V^T is formed from the 16-bit values, not INT8 codes."""
    N, D = 128, 64
    Q, K, V, dO = gaussian_head(N, D, seed=43)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=64)
    qz, O, L, delta, dOc, sdO, *_ = _full(Q, K, V, dO, sh, quant=True)
    ref = dO @ V.T
    for i in range(2):
        for j in range(2):
            t = sage.backward_tile(qz, V, dO, dOc, sdO, L, delta, i, j, sh)
            np.testing.assert_allclose(t["dP"], ref[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64], rtol=1e-13, atol=1e-13)


def test_uniform_probabilities_give_mean_dv():
    """Q = 0 makes P uniform (1/N), every P code 127, and with integer dO
    holding 127 in each block dV is the column mean of dO."""
    N, D = 128, 16
    rng = np.random.default_rng(44)
    dO = rng.integers(-120, 121, size=(N, D)).astype(np.float64)
    dO[::64, 0] = 127.0
    Q = np.zeros((N, D))
    K = rng.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32)
    qz, O, L, delta, dOc, sdO, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=True)
    assert np.all(sdO == 1.0)
    np.testing.assert_allclose(dV, np.tile(dO.mean(axis=0), (N, 1)), rtol=1e-6, atol=1e-6)


def test_q_smoothing_bias_restores_dk():
    """Quantisation off, Q-smoothing with the (dS^T 1) mu_Q^T correction gives
    the unsmoothed dK and dQ (paperlayer section 6)."""
    N, D = 128, 16
    Q, K, V, dO = gaussian_head(N, D, seed=45, q_offset=4.0)
    res = {}
    for qs in (False, True):
        sh = sage.Shape(N=N, D=D, bq=32, bkv=32, q_smooth=qs, causal=True)
        res[qs] = _full(Q, K, V, dO, sh, quant=False)[-3:]
    for a, b in zip(res[False], res[True]):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)


def test_q_smoothing_quantised_dk_close_to_exact():
    """With a large query offset the quantised dK stays accurate only because
    of the bias term; without it the error is O(1)."""
    N, D = 256, 64
    Q, K, V, dO = gaussian_head(N, D, seed=46, q_offset=4.0)
    sh = sage.Shape(N=N, D=D, bq=128, bkv=64, q_smooth=True)
    *_, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=True)
    g = fpa.backward(Q, K, V, dO, sh.scale)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(dK, g["dK"]) < 0.1
    assert rel(dQ, g["dQ"]) < 0.1


def test_subset_blocks_match_full_backward():
    N, D = 256, 32
    Q, K, V, dO = gaussian_head(N, D, seed=47)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, causal=True)
    qz, O, L, delta, dOc, sdO, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=True)
    sQ, sK, sV = sage.backward(qz, V, dO, dOc, sdO, L, delta, sh, kv_blocks=[1, 6], q_blocks=[2])
    for j in (1, 6):
        r = slice(j * 32, (j + 1) * 32)
        np.testing.assert_array_equal(sK[r], dK[r])
        np.testing.assert_array_equal(sV[r], dV[r])
    np.testing.assert_array_equal(sQ[128:192], dQ[128:192])
    assert np.isnan(sQ[:64]).all() and np.isnan(sK[:32]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_quantised_gradients_with_uneven_block_scales(causal):
    """Blocks whose magnitudes differ by up to 64x: each tile must use its own
    blocks' scales (s_Q of block i, s_K and s_V of block j, s_dO of block i)."""
    N, D = 256, 64
    Q, K, V, dO = gaussian_head(N, D, seed=48)
    ramp64 = np.repeat(2.0 ** np.arange(4), 64)[:, None]          # per 64-row block
    ramp32 = np.repeat(2.0 ** (np.arange(8) % 4 - 1), 32)[:, None]  # per 32-row block
    Q, K, V, dO = Q * ramp64 / 4, K * ramp32[::-1] / 2, V * ramp32, dO * ramp64[::-1]
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, causal=causal)
    qz, O, L, delta, dOc, sdO, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=True)
    g = fpa.backward(Q, K, V, dO, sh.scale, causal)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(O, g["O"]) < 0.05
    for ours, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        assert rel(ours, g[n]) < 0.15, n
