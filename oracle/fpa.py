"""Full-precision attention in float64 (test infrastructure; see oracle/__init__.py).

The textbook definition the SageBwd pages build on (SageBwd paper summary,
preliminaries on attention gradients; SageAttention3 write-up, Eq. 9):

  S = Q K^T * scale,  P = softmax(S) row-wise (causal: key n visible to
  query r iff n <= r),  O = P V,  L = logsumexp(S) per row,
  dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO o O),
  dS = P o (dP - delta),  dQ = scale * dS K,  dK = scale * dS^T Q.

Inputs are per-head float arrays [N, D]; everything is float64.
"""
import numpy as np


def causal_mask(n_q: int, n_k: int) -> np.ndarray:
    """True where query r may attend key n (top-left aligned: n <= r)."""
    return np.arange(n_k)[None, :] <= np.arange(n_q)[:, None]


def forward(Q, K, V, scale, causal=False):
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    S = (Q @ K.T) * scale
    if causal:
        S = np.where(causal_mask(S.shape[0], S.shape[1]), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    O = P @ V
    L = (m + np.log(l))[:, 0]
    return O, L, P


def backward(Q, K, V, dO, scale, causal=False):
    """Returns dict with dQ, dK, dV and the intermediates P, dP, dS, delta, O."""
    Q, K, V, dO = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, dO))
    O, L, P = forward(Q, K, V, scale, causal)
    dV = P.T @ dO
    dP = dO @ V.T
    delta = np.sum(dO * O, axis=1)
    dS = P * (dP - delta[:, None])
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    return {"dQ": dQ, "dK": dK, "dV": dV, "P": P, "dP": dP, "dS": dS, "delta": delta, "O": O, "L": L}
