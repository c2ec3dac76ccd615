"""CPU pins of the oracle's preprocessing step (smoothing + per-block INT8)."""
import os

import numpy as np
import pytest

from oracle import sage
from tests.oracle_cases import gaussian_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_examples.txt")


def _read_golden():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, vals = line.split(":", 1)
        cur[key] = [float(v) for v in vals.split()]
        if key == "codes":
            cases.append(cur)
            cur = {}
    return cases


@pytest.mark.parametrize("case", _read_golden())
def test_quantize_block_golden(case):
    codes, s = sage.quantize_block(np.array(case["x"]))
    assert s == case["s"][0]
    assert codes.tolist() == case["codes"]


def test_quantize_block_invariants():
    rng = np.random.default_rng(7)
    for trial in range(50):
        x = (rng.standard_normal(128 * 8) * rng.uniform(1e-3, 1e3)).astype(np.float32).astype(np.float64)
        codes, s = sage.quantize_block(x)
        a = np.max(np.abs(x))
        assert np.float32(s) == np.float32(np.float32(a) / np.float32(127))
        assert np.max(np.abs(codes)) == 127            # the extreme element maps to +-127
        assert np.all(codes == np.rint(codes))
        # reconstruction error within half a step (plus float32 rounding of x/s)
        assert np.all(np.abs(x - codes * s) <= 0.5 * s * (1 + 1e-6) + 1e-30)
        # the code is the nearest integer to the exact quotient unless the
        # quotient sits within float32 rounding of a .5 boundary
        q = x / s
        frac = np.abs(q - np.floor(q) - 0.5)
        clear = frac > 1e-4
        assert np.array_equal(codes[clear], np.clip(np.round(q[clear]), -127, 127))


def test_quantize_block_off_is_identity():
    x = np.linspace(-3, 3, 17)
    codes, s = sage.quantize_block(x, quant=False)
    assert s == 1.0 and np.array_equal(codes, x)


def test_k_mean_closed_form():
    N, D = 128, 16
    K = np.tile(np.arange(D, dtype=np.float64) - 3.5, (N, 1))     # constant columns
    Q = np.ones((N, D)); V = np.ones((N, D))
    sh = sage.Shape(N=N, D=D, bq=64, bkv=64)
    qz = sage.quantize(Q, K, V, sh)
    assert np.array_equal(qz.mu_k, np.arange(D) - 3.5)
    assert np.all(qz.K_sm == 0) and np.all(qz.Kc == 0) and np.all(qz.sK == 0)


def test_k_smoothing_centres_columns():
    Q, K, V, _ = gaussian_head(256, 32, seed=3, k_offset=4.0)
    sh = sage.Shape(N=256, D=32, bq=128, bkv=64)
    qz = sage.quantize(Q, K, V, sh)
    np.testing.assert_allclose(qz.mu_k, K.mean(axis=0), rtol=1e-6, atol=1e-7)
    # centred columns have (near) zero mean; the offset was ~4
    assert np.max(np.abs(qz.K_sm.mean(axis=0))) < 1e-5


def test_q_smoothing_blocks():
    Q, K, V, _ = gaussian_head(256, 32, seed=4, q_offset=3.0)
    sh = sage.Shape(N=256, D=32, bq=64, bkv=64, q_smooth=True)
    qz = sage.quantize(Q, K, V, sh)
    for i in range(sh.Tm):
        np.testing.assert_allclose(qz.mu_q[i], Q[i * 64:(i + 1) * 64].mean(axis=0), rtol=1e-6, atol=1e-7)
    # the Q codes quantise the centred block, whose column means are ~0
    deq = qz.Qc * np.repeat(qz.sQ, 64)[:, None]
    assert np.max(np.abs(deq.reshape(4, 64, 32).mean(axis=1))) < 0.05


def test_codes_reconstruct_inputs():
    Q, K, V, _ = gaussian_head(256, 64, seed=5)
    sh = sage.Shape(N=256, D=64, bq=128, bkv=64)
    qz = sage.quantize(Q, K, V, sh)
    deqV = qz.Vc * np.repeat(qz.sV, 64)[:, None]
    assert np.max(np.abs(deqV - V)) <= 0.5 * qz.sV.max() * 1.000001
    deqK = qz.Kc * np.repeat(qz.sK, 64)[:, None]
    assert np.max(np.abs(deqK - (K - qz.mu_k))) <= 0.5 * qz.sK.max() * 1.00001


def test_round_io_matches_numpy_fp16_and_bf16_rules():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(10000) * 10
    # fp16: numpy's float64 -> float16 cast is correctly rounded
    np.testing.assert_array_equal(sage.round_io(x, 0), x.astype(np.float16).astype(np.float64))
    # bf16: exact halfway cases round to even
    y = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130 * 1.5])
    np.testing.assert_array_equal(sage.round_io(y, 1), [1.0, 1.0 + 2 ** -6, -1.0, 2 ** -130 * 1.5])
    # bf16 of values already on the grid is the identity
    g = (np.arange(-100, 100) * 2.0 ** -5)
    np.testing.assert_array_equal(sage.round_io(g, 1), g)
