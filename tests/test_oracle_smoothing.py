"""CPU pins of the smoothing switches on offset Gaussian heads (SageBwd paper
summary, prerequisites "K-smoothing and Q-smoothing"; paperlayer section 6):
a channel offset shared by all tokens of K (or Q) inflates the per-block
INT8 scale and wastes code levels; subtracting the mean removes it, and the
method's corrections (none needed for K; the mu_Q K^T logit term and the dK
bias for Q) keep the result exact in real arithmetic.  Against full-precision
attention the error therefore falls with K-smoothing when K carries an
offset, and further with Q-smoothing when Q carries one too."""
import dataclasses

from oracle import fpa, metrics, sage
from tests.oracle_cases import gaussian_head

N, D = 512, 64


def _errors(Q, K, V, dO, ks, qs):
    sh = sage.Shape(N=N, D=D, bq=64, bkv=64, k_smooth=ks, q_smooth=qs)
    g = fpa.backward(Q, K, V, dO, sh.scale)
    r = sage.run_head(Q, K, V, dO, sh)
    return {t: metrics.rel_l2(r[t], g[t]) for t in ("O", "dQ", "dK", "dV")}


def test_k_smoothing_removes_a_k_offset():
    Q, K, V, dO = gaussian_head(N, D, seed=91, k_offset=4.0)
    none = _errors(Q, K, V, dO, False, False)
    ksm = _errors(Q, K, V, dO, True, False)
    assert ksm["O"] < none["O"] / 2 and ksm["dQ"] < none["dQ"] / 3, (none, ksm)
    assert all(ksm[t] < none[t] for t in ksm), (none, ksm)


def test_q_smoothing_removes_a_q_offset():
    Q, K, V, dO = gaussian_head(N, D, seed=91, k_offset=4.0, q_offset=3.0)
    ksm = _errors(Q, K, V, dO, True, False)
    qk = _errors(Q, K, V, dO, True, True)
    assert qk["O"] < ksm["O"] / 1.5 and qk["dK"] < ksm["dK"] / 1.5, (ksm, qk)
    assert all(qk[t] < ksm[t] for t in qk), (ksm, qk)
