"""CPU pins of the oracle's E4M3 variant (Shape.fp8): every quantised operand
takes the nearest E4M3 value of its scaled float32 quotient, with 448 in place
of 127.  The SageAttention3 write-up's INT8-versus-FP8 training table reports
the INT8 gradients as the more accurate ones; the trend pin below checks that
ordering on Gaussian heads.

The rounding itself is pinned against torch's float32 -> float8_e4m3fn
conversion (a library routine independent of the oracle) and by brute force
over every finite E4M3 bit pattern."""
import numpy as np
import pytest
import torch

from oracle import fpa, metrics, sage
from tests.oracle_cases import gaussian_head


def _torch_e4m3(x):
    """Round through torch's float8_e4m3fn (round to nearest even) and back."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _all_finite_e4m3():
    """(values, bytes) of the 254 finite E4M3 encodings (0x7f and 0xff are NaN)."""
    bits = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals, bits


def test_every_finite_encoding_round_trips():
    vals, bits = _all_finite_e4m3()
    np.testing.assert_array_equal(sage.e4m3_round(vals), vals)
    enc = sage.e4m3_bits(vals)
    # +0 and -0 both decode to 0; the oracle writes +0
    nonzero = vals != 0
    np.testing.assert_array_equal(enc[nonzero], bits[nonzero])
    assert vals.max() == sage.E4M3_MAX == 448.0
    assert np.min(vals[vals > 0]) == 2.0 ** -9


def test_rounding_matches_the_library_conversion():
    """Midpoints between neighbouring encodings (the ties), points just beside
    them, and random values across the whole range, subnormals included."""
    vals, _ = _all_finite_e4m3()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    eps = np.float64(2.0 ** -20)
    rng = np.random.default_rng(81)
    rand = rng.uniform(-448, 448, 4000) * np.exp2(-rng.integers(0, 18, 4000))
    x = np.concatenate([mids, -mids, mids * (1 + eps), mids * (1 - eps), rand]).astype(np.float32)
    np.testing.assert_array_equal(sage.e4m3_round(x.astype(np.float64)), _torch_e4m3(x))


def test_ties_go_to_the_even_mantissa():
    # between 1 (mantissa 000) and 1.125 (001): 1; between 1.125 and 1.25 (010): 1.25
    assert sage.e4m3_round(1.0625) == 1.0
    assert sage.e4m3_round(1.1875) == 1.25
    # subnormals: 2^-10 lies between 0 and 2^-9 -> 0; 3 * 2^-10 between 2^-9 and 2^-8 -> 2^-8
    assert sage.e4m3_round(2.0 ** -10) == 0.0
    assert sage.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8
    # the top binade has spacing 32: 432 is between 416 and 448 -> 448 (mantissa 110)
    assert sage.e4m3_round(432.0) == 448.0
    assert sage.e4m3_round(-(2.0 ** -6) * 1.0625) == -(2.0 ** -6)


def test_block_codes_reach_448_and_stay_within_half_a_step():
    rng = np.random.default_rng(82)
    X = (rng.standard_normal((64, 32)) * 3).astype(np.float32).astype(np.float64)
    codes, s = sage.quantize_block(X, fp8=True)
    assert s == float(np.float32(np.max(np.abs(X.astype(np.float32)))) / np.float32(448))
    assert np.max(np.abs(codes)) == 448.0
    q = (X.astype(np.float32) / np.float32(s)).astype(np.float64)
    # the spacing of E4M3 around each quotient bounds the rounding error by half of it
    _, e = np.frexp(np.where(q != 0, q, 1.0))
    step = np.exp2(np.maximum(e - 1, -6) - 3)
    assert np.all(np.abs(codes - q) <= step / 2)


def test_representable_inputs_give_exact_logits():
    """Q and K whose entries are E4M3 values times a power of two, with each
    block's maximum at 448 times it, quantise without error (the scale is that
    power of two exactly): the logits equal the full-precision ones."""
    rng = np.random.default_rng(83)
    vals, _ = _all_finite_e4m3()
    pool = vals[np.abs(vals) >= 1.0]
    N, D = 64, 32
    Q = rng.choice(pool, (N, D)) * 2.0 ** -8
    K = rng.choice(pool, (N, D)) * 2.0 ** -6
    Q[::32, 0] = 448.0 * 2.0 ** -8      # each 32-row block holds the maximum 448
    K[::32, 0] = 448.0 * 2.0 ** -6
    V = rng.standard_normal((N, D))
    sh = sage.Shape(N=N, D=D, bq=32, bkv=32, k_smooth=False, fp8=True)
    qz = sage.quantize(Q, K, V, sh)
    np.testing.assert_array_equal(qz.sQ, 2.0 ** -8)
    np.testing.assert_array_equal(qz.sK, 2.0 ** -6)
    for i in range(sh.Tm):
        for j in range(sh.Tn):
            S = sage.logits(qz, i, j, sh)
            ref = Q[i * 32:(i + 1) * 32] @ K[j * 32:(j + 1) * 32].T * sh.scale
            np.testing.assert_allclose(S, ref, rtol=1e-15, atol=0)


def test_forward_p_codes_top_out_at_448():
    """At each row's maximum P~ / s_P = exp(rm - m) / (exp(rm - m) / 448) = 448."""
    N, D = 128, 32
    Q, K, V, _ = gaussian_head(N, D, seed=84, sigma=1.5)
    sh = sage.Shape(N=N, D=D, bq=64, bkv=32, fp8=True)
    qz = sage.quantize(Q, K, V, sh)
    S = sage.logits(qz, 0, 1, sh)
    rm = S.max(axis=1)
    m = np.maximum(rm, rm - 0.7)           # m = rm: every row's maximum is exp(0) = 1
    sP, codes = sage.per_token_p_quant(np.exp(S - m[:, None]), rm, m, fp8=True)
    np.testing.assert_array_equal(codes.max(axis=1), 448.0)
    np.testing.assert_array_equal(sP, np.float32(1) / np.float32(448))
    np.testing.assert_array_equal(sage.e4m3_round(codes), codes)


def test_quant_off_variant_is_exact_attention():
    N, D = 64, 16
    Q, K, V, dO = gaussian_head(N, D, seed=85, sigma=1.0)
    sh = sage.Shape(N=N, D=D, bq=32, bkv=16, causal=True, fp8=True)
    r = sage.run_head(Q, K, V, dO, sh, quant=False)
    O_ref = fpa.forward(Q, K, V, sh.scale, True)[0]
    g = fpa.backward(Q, K, V, dO, sh.scale, True)
    np.testing.assert_allclose(r["O"], O_ref, rtol=1e-10, atol=1e-12)
    for n in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(r[n], g[n], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [86, 87])
def test_int8_gradients_more_accurate_than_fp8(seed):
    """The direction of the INT8-versus-FP8 training table: against
    full-precision gradients, INT8 SageBwd has the lower relative L1 error and
    the higher cosine similarity on dQ, dK and dV."""
    N, D = 256, 64
    Q, K, V, dO = gaussian_head(N, D, seed=seed, sigma=1.0)
    g = fpa.backward(Q, K, V, dO, 1 / np.sqrt(D), False)
    res = {}
    for fp8 in (False, True):
        sh = sage.Shape(N=N, D=D, bq=64, bkv=64, fp8=fp8)
        res[fp8] = sage.run_head(Q, K, V, dO, sh)
    for n in ("dQ", "dK", "dV"):
        l1 = {f: metrics.rel_l1(res[f][n], g[n]) for f in (False, True)}
        cs = {f: metrics.cos_sim(res[f][n], g[n]) for f in (False, True)}
        assert l1[False] < l1[True], (n, l1)
        assert cs[False] > cs[True], (n, cs)


def test_variant_rejects_the_int8_only_switches():
    with pytest.raises(ValueError):
        sage.Shape(N=64, D=16, bq=32, bkv=32, fp8=True, dp_int8=True)
    with pytest.raises(ValueError):
        sage.Shape(N=64, D=16, bq=32, bkv=32, fp8=True, p_static=True)
