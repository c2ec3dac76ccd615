"""The quantisation kernels round x/s to float32 without a division per
element: r = RN64(1/s) once per block, then RN32(RN64(x * r)).  That equals
the correctly rounded float32 quotient RN32(x/s) that the codes are defined
on, because RN64(x * r) is within 2^-52 (relative) of x/s while a quotient of
two float32 values is never within 2^-49 of a float32 rounding midpoint (a
midpoint has 25 significant bits, so x - m*s is a nonzero multiple of a power
of two at most 2^-49 of x).  Checked here with numpy's IEEE arithmetic on
random pairs, on quotients placed next to midpoints, and on the block-scale
shape the kernels use (s = RN32(max|x| / 127), |x| <= max|x|)."""
import numpy as np


def _fast(x, s):
    r = np.float64(1.0) / s.astype(np.float64)
    return (x.astype(np.float64) * r).astype(np.float32)


def _exact(x, s):
    return (x / s).astype(np.float32)     # float32 / float32: correctly rounded


def test_random_pairs_over_the_range():
    rng = np.random.default_rng(7)
    n = 2_000_000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
    s = (rng.random(n) * np.exp2(rng.integers(-60, 60, n)) + 1e-30).astype(np.float32)
    np.testing.assert_array_equal(_fast(x, s), _exact(x, s))


def test_block_scales_and_codes():
    rng = np.random.default_rng(11)
    for q in (127.0, 448.0):
        blocks = rng.standard_normal((4000, 512)).astype(np.float32) * np.float32(3.0)
        a = np.abs(blocks).max(axis=1)
        s = (a / np.float32(q)).astype(np.float32)[:, None]
        np.testing.assert_array_equal(_fast(blocks, np.broadcast_to(s, blocks.shape)),
                                      _exact(blocks, np.broadcast_to(s, blocks.shape)))


def test_quotients_next_to_rounding_midpoints():
    """x chosen so that x/s lands as close to a float32 midpoint as float32
    x allows: x = RN32(m*s) for midpoints m of codes' range, and its float32
    neighbours."""
    rng = np.random.default_rng(3)
    s = (rng.random(200_000) * 2 + 0.5).astype(np.float32) * np.float32(2.0 ** -7)
    k = rng.integers(-127, 127, s.size).astype(np.float64)
    frac = rng.random(s.size)
    m = k + frac                                     # a value in the code range
    m32 = m.astype(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(m32).astype(np.float32)).astype(np.float64)
    mid = m32 + ulp / 2                               # a float32 midpoint
    x0 = (mid * s.astype(np.float64)).astype(np.float32)
    for dx in (-2, -1, 0, 1, 2):
        x = np.nextafter(x0, np.float32(np.inf) if dx > 0 else np.float32(-np.inf)) if dx else x0
        for _ in range(abs(dx) - 1):
            x = np.nextafter(x, np.float32(np.inf) if dx > 0 else np.float32(-np.inf))
        np.testing.assert_array_equal(_fast(x, s), _exact(x, s))


def test_subnormal_inputs_and_scales():
    tiny = np.float32(1.4e-45)
    x = np.array([tiny, -tiny, tiny * 7, np.float32(1e-39), np.float32(-3e-40), np.float32(0.0)], np.float32)
    for s in (np.float32(1e-42), np.float32(3e-39), np.float32(1.0), np.float32(1e-20)):
        ss = np.full_like(x, s)
        np.testing.assert_array_equal(_fast(x, ss), _exact(x, ss))
