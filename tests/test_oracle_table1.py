"""The oracle against the SageBwd paper's Table 1 (sigma sweep).

The table's shapes are not given; the sigma-sweep workload (d = 128,
non-causal, K-smoothing on, Q-smoothing off) is run here at a reduced size
(2 heads of N = 1024).  What is pinned:

* the trend: every tensor's error grows with sigma (from sigma = 3 on, and
  sigma = 5 above sigma = 1), dQ and dK degrade far faster than O and dV,
  O tracks dV and dQ tracks dK;
* for sigma >= 3, where the INT8 logits dominate the error, each rel-L2 lies
  within a factor 1.5 of the table's value.

At sigma = 1 the per-tile quantisation of P and dS in the backward pass (one
scale per 128 x 64 tile) dominates dQ, dK and dV; those errors come out about
3x the table's, so "O tracks dV" (the table's pattern at every sigma) holds
here only from sigma = 3 on.  tests/test_oracle_granularity.py pins the account: the same backward
with per-row P and dS scales reproduces the table's sigma = 1 row, and
smaller tiles close the gap monotonically while O stays put.
"""
import os

import numpy as np
import pytest

from bit_trainable_attention_block_amd import workloads as wl
from oracle import fpa, metrics, sage

TABLE = os.path.join(os.path.dirname(__file__), "golden", "table1_sigma_sweep.txt")
NAMES = ("O", "dQ", "dK", "dV")


def _pages():
    rows = {}
    for line in open(TABLE):
        if line.strip() and not line.startswith("#"):
            v = [float(x) for x in line.split()]
            rows[v[0]] = {n: (v[1 + 2 * k], v[2 + 2 * k]) for k, n in enumerate(NAMES)}
    return rows


@pytest.fixture(scope="module")
def sweep():
    out = {}
    for c in wl.C4:
        cfg = c.replace(N=1024, H=2)
        x = wl.generate(cfg)
        sh = sage.Shape.of(cfg)
        ours = {n: [] for n in NAMES}
        refs = {n: [] for n in NAMES}
        for h in range(cfg.H):
            Q, K, V, dO = (x[n]["f32"][0, h].astype(np.float64) for n in ("q", "k", "v", "do"))
            r = sage.run_head(Q, K, V, dO, sh)
            g = fpa.backward(Q, K, V, dO, sh.scale)
            for n in NAMES:
                ours[n].append(r[n])
                refs[n].append(g[n])
        out[cfg.sigma] = {n: metrics.all_metrics(np.stack(ours[n]), np.stack(refs[n])) for n in NAMES}
    return out


def test_errors_grow_with_sigma(sweep):
    for n in NAMES:
        rel = [sweep[s][n]["rel_l2"] for s in wl.SIGMAS]
        cos = [sweep[s][n]["cos"] for s in wl.SIGMAS]
        assert rel[1] < rel[2] < rel[3] <= rel[4] * 1.02, (n, rel)
        assert rel[0] < rel[2], (n, rel)
        assert cos[1] > cos[2] > cos[3] >= cos[4] - 1e-3, (n, cos)


def test_gradient_errors_concentrate_in_dq_dk(sweep):
    for s in (5.0, 8.0, 10.0):
        m = sweep[s]
        assert min(m["dQ"]["rel_l2"], m["dK"]["rel_l2"]) > 2.5 * max(m["O"]["rel_l2"], m["dV"]["rel_l2"])
    m = sweep[10.0]
    assert min(m["dQ"]["rel_l2"], m["dK"]["rel_l2"]) > 4 * max(m["O"]["rel_l2"], m["dV"]["rel_l2"])
    for s in wl.SIGMAS:
        m = sweep[s]
        assert abs(m["dQ"]["rel_l2"] / m["dK"]["rel_l2"] - 1) < 0.1
        if s >= 3:
            assert abs(m["O"]["rel_l2"] / m["dV"]["rel_l2"] - 1) < 0.1


def test_values_near_table_where_logits_dominate(sweep):
    pages = _pages()
    for s in (3.0, 5.0, 8.0, 10.0):
        for n in NAMES:
            ours = sweep[s][n]["rel_l2"]
            ref = pages[s][n][1]
            assert ref / 1.5 < ours < ref * 1.5, (s, n, ours, ref)
