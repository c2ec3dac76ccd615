"""CPU pins of the oracle's INT8-dP ablation (Shape.dp_int8): dP = dO V^T
formed from the per-block INT8 codes of dO and V instead of the 16-bit values.
The SageAttention3 write-up (Table 1c) compares the two choices and keeps
FP16; SageBwd keeps dP in 16-bit for the same reason (its dS argument)."""
import dataclasses

import numpy as np
import pytest

from oracle import fpa, metrics, sage
from tests.oracle_cases import gaussian_head


def _full(Q, K, V, dO, sh, quant):
    qz = sage.quantize(Q, K, V, sh, quant)
    O, L = sage.forward(qz, sh, quant)
    delta, dOc, sdO = sage.backward_pre(O, dO, sh, quant)
    dQ, dK, dV = sage.backward(qz, V, dO, dOc, sdO, L, delta, sh, quant)
    return qz, O, L, delta, dOc, sdO, dQ, dK, dV


@pytest.mark.parametrize("causal", [False, True])
def test_quant_off_ablation_is_the_exact_gradient(causal):
    """With quantisation off the codes are the values and the scales 1, so the
    ablation reduces to exact attention gradients."""
    N, D = 64, 16
    Q, K, V, dO = gaussian_head(N, D, seed=71, sigma=1.2)
    sh = sage.Shape(N=N, D=D, bq=32, bkv=32, causal=causal, dp_int8=True)
    *_, dQ, dK, dV = _full(Q, K, V, dO, sh, quant=False)
    g = fpa.backward(Q, K, V, dO, sh.scale, causal)
    for ours, ref in ((dQ, g["dQ"]), (dK, g["dK"]), (dV, g["dV"])):
        np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-12)


def test_int8_dp_within_the_quantisation_error_bound():
    """Each block code satisfies |x - code * s| <= s / 2 (s = max|X| / 127,
    round to nearest), so with dO = dO^ s_dO + e1 and V = V^ s_V + e2:
      |dO^ V^^T s_dO s_V - dO V^T| <= sum_d (s_dO/2 |V| + s_V/2 |dO| + s_dO s_V / 4)
    elementwise.  A transposed operand, a missing or misplaced scale, or the
    wrong block's scale breaks it; the bound is also shown not to be loose."""
    N, D = 128, 64
    Q, K, V, dO = gaussian_head(N, D, seed=72, sigma=1.0)
    dO = dO * np.linspace(0.2, 3.0, D)[None, :]    # uneven channels: the scales differ per block
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, dp_int8=True)
    qz, O, L, delta, dOc, sdO, *_ = _full(Q, K, V, dO, sh, quant=True)
    ratios = []
    for i in range(sh.Tm):
        for j in range(sh.Tn):
            rows = slice(i * sh.bq, (i + 1) * sh.bq)
            keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
            # the block scales from their definition, max|X| / 127
            s_do = np.max(np.abs(dO[rows])) / 127.0
            s_v = np.max(np.abs(V[keys])) / 127.0
            bound = (np.abs(V[keys]).sum(1)[None, :] * s_do / 2 + np.abs(dO[rows]).sum(1)[:, None] * s_v / 2
                     + D * s_do * s_v / 4) * (1 + 1e-5)
            t = sage.backward_tile(qz, V, dO, dOc, sdO, L, delta, i, j, sh)
            err = np.abs(t["dP"] - dO[rows] @ V[keys].T)
            assert np.all(err <= bound), (i, j, float(np.max(err / bound)))
            ratios.append(np.median(err / bound))
    assert 0.01 < float(np.median(ratios)) < 0.5


def test_ablation_changes_only_the_dp_path():
    """dV does not depend on dP: identical in both modes.  dQ and dK do."""
    N, D = 128, 64
    Q, K, V, dO = gaussian_head(N, D, seed=73)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=64)
    *_, dQ0, dK0, dV0 = _full(Q, K, V, dO, sh, quant=True)
    *_, dQ1, dK1, dV1 = _full(Q, K, V, dO, dataclasses.replace(sh, dp_int8=True), quant=True)
    np.testing.assert_array_equal(dV0, dV1)
    assert not np.array_equal(dQ0, dQ1) and not np.array_equal(dK0, dK1)


def test_int8_dp_degrades_dq_dk_like_table_1c():
    """SageAttention3 write-up, Table 1c: dO V^T in INT8 gives a lower cosine
    and a larger L1 error than FP16 (97.47% vs 99.77%, L1 0.171 vs 0.039 on
    the pages' setup, whose shapes and data are not stated).  Against
    full-precision attention, dQ and dK here move the same way: slightly on
    iid Gaussian heads, where the per-tile dS codes dominate the error, and
    by a wide margin once a few channels of dO and V are large (as in real
    gradients), since a block's INT8 scale then follows those channels."""
    N, D = 512, 64
    for outlier, min_ratio in ((1.0, 1.01), (8.0, 1.3)):
        Q, K, V, dO = gaussian_head(N, D, seed=74)
        w = np.ones(D)
        w[:2] = outlier
        dO, V = dO * w[None, :], V * w[None, ::-1]
        sh = sage.Shape(N=N, D=D, bq=64, bkv=64)
        g = fpa.backward(Q, K, V, dO, sh.scale)
        *_, dQ0, dK0, _ = _full(Q, K, V, dO, sh, quant=True)
        *_, dQ1, dK1, _ = _full(Q, K, V, dO, dataclasses.replace(sh, dp_int8=True), quant=True)
        for ours16, ours8, ref in ((dQ0, dQ1, g["dQ"]), (dK0, dK1, g["dK"])):
            m16, m8 = metrics.all_metrics(ours16, ref), metrics.all_metrics(ours8, ref)
            assert m8["cos"] < m16["cos"], (outlier, m16, m8)
            assert m8["rel_l1"] > min_ratio * m16["rel_l1"], (outlier, m16, m8)
