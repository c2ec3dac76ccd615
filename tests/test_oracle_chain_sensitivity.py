"""Why the whole-chain comparison takes a looser bar than the per-call one.

The forward stores O rounded to the 16-bit I/O dtype, and delta =
rowsum(dO o O) is taken from the stored O.  An O element whose unrounded
value lies within a hair of a rounding midpoint can legitimately round either
way (the GPU sums in another order and takes exp2 to an ulp).  A flip moves
delta by one 16-bit ulp of O times dO.  That shifts a row of dS, and it can
change a whole tile's dS scale and codes.

The oracle's own chain is run on the small Q-smoothing case of the GPU tests,
once as is and once with the few O elements closest to a bf16 midpoint
rounded the other way.  Four such flips (O's rel-L2 5e-5, below what the GPU
and the oracle differ by on that case) move dQ and dK by more than 1e-3.  dV,
which does not depend on delta, stays put.  So the chain comparison cannot be
held to the per-call 1e-3, and the GPU tests use 5e-3 for it.
"""
import numpy as np
import pytest

from bit_trainable_attention_block_amd import workloads as wl
from oracle import metrics, sage

CASE = wl.Config("n256_d128_qsmooth", 9, 1, 2, 256, 128, wl.BF16, 128, 64, causal=False, k_smooth=True,
                 q_smooth=True, sigma=3.0, qk_norm=False, k_offset_sigma=1.5)


def _forward_unrounded(qz, sh, monkeypatch):
    """O before and after the rounding to bf16, and L."""
    seen = {}
    real = sage.round_io

    def spy(v, dtype):
        seen["pre"] = np.array(v, dtype=np.float64)
        return real(v, dtype)

    monkeypatch.setattr(sage, "round_io", spy)
    O, L = sage.forward(qz, sh)
    monkeypatch.setattr(sage, "round_io", real)
    return seen["pre"], O, L


def _flip_nearest_midpoints(pre, O, k):
    """O with its k elements nearest a bf16 rounding midpoint rounded the
    other way (one bf16 ulp toward the unrounded value)."""
    p, o = pre.ravel(), O.ravel().copy()
    _, e = np.frexp(np.where(p != 0, p, 1.0))
    ulp = np.exp2(e - 8.0)                       # bf16 keeps 8 significant bits
    frac = np.abs(p - o) / ulp                   # 0.5 on a midpoint
    idx = np.argsort(-frac)[:k]
    o[idx] += np.sign(p[idx] - o[idx]) * ulp[idx]
    return o.reshape(O.shape), frac[idx].min()


def test_four_rounding_flips_of_o_move_the_chain_by_1e3(monkeypatch):
    x = wl.generate(CASE)
    sh = sage.Shape.of(CASE)
    Q, K, V, dO = (x[n]["f32"][0, 0].astype(np.float64) for n in ("q", "k", "v", "do"))
    qz = sage.quantize(Q, K, V, sh)
    pre, O, L = _forward_unrounded(qz, sh, monkeypatch)
    # the rounded O the oracle stores is the unrounded one to within half an ulp
    np.testing.assert_array_equal(O, sage.round_io(pre, sh.dtype))

    def grads(Ox):
        delta, dOc, sdO = sage.backward_pre(Ox, dO, sh)
        return sage.backward(qz, V, dO, dOc, sdO, L, delta, sh)

    base = grads(O)
    Of, nearest = _flip_nearest_midpoints(pre, O, 4)
    assert nearest > 0.4999                       # each flip is within 1e-4 ulp of a midpoint
    assert metrics.rel_l2(Of, O) < 1e-4
    dQ, dK, dV = grads(Of)
    assert metrics.rel_l2(dQ, base[0]) > 1e-3
    assert metrics.rel_l2(dK, base[1]) > 1e-3
    assert metrics.rel_l2(dV, base[2]) == 0.0     # dV does not depend on delta
    assert metrics.rel_l2(dK, base[1]) < 5e-3     # ... and the chain bar covers it
