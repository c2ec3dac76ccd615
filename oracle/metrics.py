"""Accuracy metrics (test infrastructure; see oracle/__init__.py).

The SageAttention3 write-up defines its error metrics in its table of
quantisation-error metrics: cosine similarity sum(O O') / sqrt(sum O^2 sum
O'^2), a relative L1 error (the formula is cut off in the page text; read as
sum|O - O'| / sum|O|, the relative form the ratio suggests), and RMSE
sqrt(mean (O - O')^2).  The SageBwd paper's Tables 1 and 2 add the relative
L2 error ||O - O'||_2 / ||O||_2.  All are computed in float64 over the
flattened tensors, with the second argument as the reference.
"""
import numpy as np


def _flat(x):
    return np.asarray(x, dtype=np.float64).ravel()


def cos_sim(x, ref):
    a, b = _flat(x), _flat(ref)
    den = np.sqrt(np.dot(a, a) * np.dot(b, b))
    return float(np.dot(a, b) / den) if den > 0 else float(np.array_equal(a, b))


def rel_l2(x, ref):
    a, b = _flat(x), _flat(ref)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def rel_l1(x, ref):
    a, b = _flat(x), _flat(ref)
    sb = np.sum(np.abs(b))
    return float(np.sum(np.abs(a - b)) / sb) if sb > 0 else float(np.sum(np.abs(a)))


def rmse(x, ref):
    a, b = _flat(x), _flat(ref)
    return float(np.sqrt(np.mean((a - b) ** 2))) if a.size else 0.0


def all_metrics(x, ref):
    return {"cos": cos_sim(x, ref), "rel_l2": rel_l2(x, ref), "rel_l1": rel_l1(x, ref), "rmse": rmse(x, ref)}
